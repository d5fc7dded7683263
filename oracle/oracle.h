/* oracle.h -- plain CPU reference for the quantized MoE feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header or table with the GPU library; the two meet only in the bytes the
 * seeded input generators produce.
 *
 * Everything is the plain definition written out: weights are decoded to
 * their exact values, every dot product is summed sequentially in double
 * precision, and results are rounded to fp32 once at the end.
 */
#ifndef MD_ORACLE_H
#define MD_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { OR_Q8_0 = 1, OR_Q4_0 = 2, OR_I8_ROW = 3, OR_I4_ROW = 4, OR_Q4_1 = 5, OR_I2_ROW = 6 };
enum { OR_X_F32 = 0, OR_X_BF16 = 1 };
enum { OR_ACT_GELU_TANH = 0, OR_ACT_SILU = 1 };
enum { OR_OK = 0, OR_EINVAL = 1, OR_ENONFINITE = 2, OR_EMISSING = 3 };

/* A quantized matrix in the canonical layout (rows x cols, row-major). */
typedef struct {
    int32_t fmt;
    int32_t rows, cols;
    const uint8_t *data;     /* rows * row_bytes; NULL = not supplied       */
    const float *scales;     /* per-row fp32 scales for the *_ROW formats  */
} or_qmat;

/* One MoE layer.  gate/up/down point at arrays of E matrices; an entry whose
 * data is NULL is an expert the caller did not materialise (selecting it is
 * an error, OR_EMISSING). */
typedef struct {
    int32_t H, F, E, k, act;
    const float *Wr;         /* E x H                                       */
    const float *bias;       /* E, or NULL                                  */
    const or_qmat *gate, *up, *down;
    int32_t has_shared;
    or_qmat sh_gate, sh_up, sh_down;
} or_moe;

int or_set_threads(int n);
int or_get_threads(void);
int or_row_bytes(int fmt, int cols);

/* Decode one row of K weights to their exact values. */
int or_decode_row(int fmt, const uint8_t *row, float scale, int K, double *w);

/* y[b][r] = fl32(sum_c w[r][c] x[b][c]);  S[b][r] = sum_c |w[r][c] x[b][c]|. */
int or_qgemv(const or_qmat *W, int xtype, const void *x, int B, float *y, double *S);

/* Router: logits, top-k (descending logit, exact ties to the lower expert
 * index) and softmax gates over the selected k.  logits/margin may be NULL.
 * margin[t] = (k-th selected logit) - (best unselected logit), +inf if k==E. */
int or_route_topk(const float *x, int T, int H, const float *Wr, const float *bias,
                  int E, int k, int32_t *idx, float *gates, float *logits, float *margin);

/* Dense gated FFN: y = down( act(gate x) * (up x) ); S as for the last GEMV. */
int or_ffn(const or_qmat *gate, const or_qmat *up, const or_qmat *down, int act,
           const float *x, int T, float *y, double *S);

/* The whole layer: route, run the k selected experts, weight by the gates,
 * add the shared expert.  idx/gates are written (T x k); S is the tolerance
 * basis (T x H). */
int or_moe_forward(const or_moe *L, const float *x, int T, float *y,
                   int32_t *idx, float *gates, double *S);

#ifdef __cplusplus
}
#endif
#endif
