// la_launch.h -- internal launchers behind the C ABI (not exported).
//
// Sequence split shared by the causal and global forms: each (b, h) pair -- "bh", 0..B*H-1 --
// is cut into P segments of L tokens (L a multiple of the chunk; the last segment may be
// shorter). Per-segment partial states live in a float32 workspace of B*H*P slots, slot
// (bh, p) at offset (bh * P + p) * E floats with E = d * d_v + d: the d x d_v state first
// (row-major, rows = key features), then the d-vector z.
#pragma once

#include <hip/hip_runtime.h>

namespace la {

// Variant flags (the same bits as the ABI's LA_PHI_IDENTITY and LA_UNNORMALIZED).
constexpr int F_IDENTITY = 1; // q and k are taken as already-mapped features (phi = identity)
constexpr int F_UNNORM = 2;   // out = phi(q)^T S, no division by phi(q)^T z

// ---- matrix-core family: bf16, d == d_v in {64, 128}, chunk 64 ---------------------------
// Segment sums dS = phi(K_seg)^T V_seg, dz = phi(K_seg)^T 1 of segments p < nseg of every
// head, written to dstS + (bh * P + p) * sstride and dstz + (bh * P + p) * zstride.
// gamma (optional, device [H] float32): per-head decay of the carried state; the sums are then
// decayed to each segment's last token. S0/z0 (optional, with nseg < P): the initial state of
// every head ([BH, D, D], [BH, D]), copied into slot nseg of the head on the way.
hipError_t agg_mfma(int D, int flags, const void *k, const void *v, float *dstS, float *dstz,
                    long sstride, long zstride, int BH, int N, int L, int nseg, int P,
                    const float *gamma, int H, const float *S0, const float *z0, hipStream_t st);
// Where the causal kernels find the state before each segment (pm):
//   0        preS/prez + (bh * P + p) * stride holds it (zero state if preS is null);
//   PM_SUMS  preS/prez is the workspace written by agg_mfma with nseg = P - 1 (slot stride
//            pstride == pzstride): segment p adds the sums of segments 0..p-1 itself, in
//            order, to the initial state in slot P - 1 (PM_INIT) or to zero;
//   PM_XCD   (with PM_SUMS, BH % 8 == 0) every segment of a head runs on the same XCD, so the
//            head's sums are fetched into one L2.
constexpr int PM_SUMS = 1, PM_INIT = 2, PM_XCD = 4;
// Causal outputs of all P segments. The last segment writes the final state to Sout/zout when
// they are non-null.
hipError_t causal_mfma(int D, int flags, const void *q, const void *k, const void *v, void *out,
                       const float *preS, const float *prez, long pstride, long pzstride, int pm,
                       float *Sout, float *zout, int BH, int N, int L, int P, const float *gamma,
                       int H, hipStream_t st);
// Random-feature forms of the two: q, k are mapped to exp(W x - |x|^2 / 2) / sqrt(D) while
// staged (W bf16 [D][D]; m = d = d_v = D); the attention is the identity-map form over them.
hipError_t agg_rf_mfma(int D, const void *k, const void *v, const void *W, float *dstS, float *dstz,
                       long sstride, long zstride, int BH, int N, int L, int nseg, int P,
                       const float *S0, const float *z0, hipStream_t st);
hipError_t causal_rf_mfma(int D, int flags, const void *q, const void *k, const void *v,
                          const void *W, void *out, const float *preS, const float *prez,
                          long pstride, long pzstride, int pm, float *Sout, float *zout, int BH,
                          int N, int L, int P, hipStream_t st);
// Global read: out = phi(Q) S / phi(Q) z for every token, S/z per head ([BH, D, D], [BH, D]).
hipError_t global_read_mfma(int D, int flags, const void *q, void *out, const float *S,
                            const float *z, int BH, int N, int L, int P, hipStream_t st);

// ---- float32 matrix-core family: d = d_v in {64, 128}, float32 inputs, chunks of 32 -------
// The same three roles as above, with the optional decay (no in-kernel feature map); the global
// read takes its own split of the rows.
hipError_t agg_mfma32(int D, int flags, const void *k, const void *v, float *dstS, float *dstz,
                      long sstride, long zstride, int BH, int N, int L, int nseg, int P,
                      const float *gamma, int H, hipStream_t st);
hipError_t causal_mfma32(int D, int flags, const void *q, const void *k, const void *v, void *out,
                         const float *preS, const float *prez, long pstride, long pzstride,
                         float *Sout, float *zout, int BH, int N, int L, int P, const float *gamma,
                         int H, hipStream_t st);
hipError_t global_read_mfma32(int D, int flags, const void *q, void *out, const float *S,
                              const float *z, int BH, int N, hipStream_t st);

// ---- vector-ALU family: any d, d_v in {16, 32, 64, 128}, float32 or bf16, chunk 16/32 ----
hipError_t agg_valu(bool bf16, int flags, const void *k, const void *v, float *dstS, float *dstz,
                    long sstride, long zstride, int BH, int N, int d, int dv, int chunk, int L,
                    int nseg, int P, const float *gamma, int H, hipStream_t st);
// Segment p of head bh starts from the state in slot bh * pslots + min(p, pslots - 1) of
// preS/prez (zero state if preS is null). causal = false gives the global read (pslots = 1:
// every segment reads the head's full state; nothing is updated).
hipError_t out_valu(bool bf16, bool causal, int flags, const void *q, const void *k, const void *v,
                    void *out, const float *preS, const float *prez, long pstride,
                    long pzstride, int pslots, float *Sout, float *zout, int BH, int N, int d,
                    int dv, int chunk, int L, int P, const float *gamma, int H, hipStream_t st);

// Dynamic LDS bytes of the vector-ALU kernels for this shape.
size_t valu_lds_bytes(int d, int dv, int chunk);
// The causal form of a short sequence (short_ok: N <= 64, d and d_v in {16, 32}) as one chunk, one
// workgroup per head, no decay: out, and the final state into S, z when S is non-null; S0, z0
// (optional, may be S, z) the state before token 0.
bool short_ok(int N, int d, int dv);
hipError_t short_causal(bool bf16, int flags, const void *q, const void *k, const void *v, void *out,
                        const float *S0, const float *z0, float *S, float *z, int BH, int N, int d,
                        int dv, hipStream_t st);

// ---- segment joins -----------------------------------------------------------------------
// In place: slots 0..P-2 hold segment sums on entry; on return slot p (0..P-1) holds the
// state before segment p (the sum of earlier segments plus the optional initial state). With a
// decay gamma (device [H]) the running state is scaled by gamma^L before each segment's sum is
// added (all scanned segments hold L tokens).
hipError_t seg_exclusive_scan(float *ws, const float *S0, const float *z0, int BH, int P,
                              int d, int dv, const float *gamma, int H, int L, hipStream_t st);
// S, z = sum of the P slots (fixed order p = 0..P-1).
hipError_t seg_total(const float *ws, float *S, float *z, int BH, int P, int d, int dv,
                     hipStream_t st);

// ---- positive random features ------------------------------------------------------------
// f[i][r] = exp(W[r] . x[i] - |x[i]|^2 / 2) / sqrt(m) for rows i, projections r < m. The
// matrix-core kernel serves bf16 with rf_mfma_ok(d, m); a float32-arithmetic kernel takes any
// d <= rf_max_d() and m.
bool rf_mfma_ok(bool bf16, int d, int m);
int rf_max_d();
hipError_t rf_features(bool bf16, const void *x, const void *W, void *f, long rows, int d, int m,
                       hipStream_t st);

// ---- decode ------------------------------------------------------------------------------
hipError_t decode_step(bool bf16, int flags, const void *q, const void *k, const void *v, void *out,
                       float *S, float *z, int BH, int d, int dv, const float *gamma, int H,
                       hipStream_t st);

} // namespace la
