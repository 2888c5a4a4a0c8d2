/*
 * CPU oracle of the quantised MoE layer.  TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct C implementation of what the MoE layer
 * computes, used to check the HIP path.  Only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark may load it; the product library
 * never does.  It shares no code, header or constant with the HIP path.
 *
 * Sources (the pages describe the method only in prose; no code is printed):
 *  - GeekNews #31297 "Show HN: running GLM 5.2 on a slow computer"
 *    (news.hada.io), section "implemented features": DeepSeek-V3-style
 *    sigmoid router with noaux_tc, routed_scaling_factor and a shared
 *    expert; integer-dot kernels on Q8_0-style int8 activations; int8 /
 *    packed int4 / packed int2 weights with per-row scales, dequant-on-use;
 *    batch-union MoE for prefill and MTP verification.
 *  - wpnews.pro "Colibri - GLM-5.2 (744B MoE) on 25GB RAM in one pure C
 *    file", model spec table: 256 experts per layer, 8 active + 1 shared;
 *    kernel table: Q8_0-style int8, packed int4 dequant-on-use.
 * Where the pages are silent the oracle takes one stated reading; each such
 * point is marked "reading:" at the function that takes it.
 *
 * Every floating-point step is fp64 unless a step says otherwise; loops run
 * in ascending index order; OpenMP (when enabled) splits only independent
 * outputs, so results do not depend on the thread count.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

typedef struct {
    int32_t hidden;       /* H */
    int32_t inter;        /* I, expert intermediate size */
    int32_t n_experts;    /* E routed experts */
    int32_t n_group;      /* G expert groups (contiguous index ranges of E/G) */
    int32_t topk_group;   /* groups kept per token */
    int32_t top_k;        /* k experts per token */
    int32_t n_shared;     /* 0 or 1 shared expert */
    int32_t wbits;        /* 2, 4 or 8 */
    double  rsf;          /* routed_scaling_factor */
    double  top_p;        /* adaptive expert top-p threshold in (0, 1); 0 or >= 1: off */
} oracle_shape;

/* One expert: packed codes, row-major [rows][rows_bytes], plus fp32 per-row
 * scales.  gate/up: rows = I over in = H; down: rows = H over in = I. */
typedef struct {
    const uint8_t *gate, *up, *down;
    const float *gate_s, *up_s, *down_s;
} oracle_expert;

/* signed code j of a packed row (two's complement; int4: element 2m is the
 * low nibble of byte m; int2: element 4m+i sits at bits 2i..2i+1) */
int oracle_code(int wbits, const uint8_t *row, int j);
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

int oracle_route(const oracle_shape *sh, const float *x, int T, const float *gate_w,
                 const float *bias, int32_t *idx, float *w, double *margins);
void oracle_router_scores(const oracle_shape *sh, const float *x, const float *gate_w,
                          const float *bias, double *s, double *c);
void oracle_quant_act(const float *x, int T, int D, int8_t *q, float *d);
void oracle_block_dots(int wbits, const uint8_t *codes, int rows, int D, const int8_t *q,
                       int T, int32_t *out);
void oracle_matvec(int wbits, const uint8_t *codes, const float *s_w, int rows, int D,
                   const int8_t *q, const float *d, int T, float *y);
void oracle_dequant_matmul(int wbits, const uint8_t *codes, const float *s_w, int rows, int D,
                           const int8_t *q, const float *d, int T, double *y);
int oracle_expert_ffn(const oracle_shape *sh, const oracle_expert *ex, const int8_t *q,
                      const float *d, int T, float *y, int8_t *qh, float *dh);
int oracle_layer_forward(const oracle_shape *sh, const float *x, int T, const float *gate_w,
                         const float *bias, const oracle_expert *const *routed,
                         const oracle_expert *shared, float *y, int32_t *idx, float *w);
int oracle_combine(const oracle_shape *sh, int T, const float *w, const float *y_slots,
                   const float *y_shared, float *out);
void oracle_rmsnorm(const float *x, const float *g, double eps, int T, int H, float *out);
int oracle_permute(const int32_t *idx, int T, int k, int E, int32_t *perm, int32_t *off,
                   int32_t *inv);
/* MTP draft verification of B sequences of D drafts over a vocabulary of V:
 * draft [B][D], p_logits [B][D+1][V] (target), q_logits [B][D][V] (draft
 * model), uniforms u [B][D+1] in [0, 1); n_acc [B] drafts kept, next [B] the
 * token emitted after them; margins [B] (nullable) the smallest relative
 * distance of any sampled decision from its boundary. */
int oracle_mtp_accept(int B, int D, int V, const int32_t *draft, const float *p_logits,
                      const float *q_logits, double tau, const double *u, int32_t *n_acc,
                      int32_t *next, double *margins);

#endif
