// Internal kernel launchers (host side). Not part of the C ABI.
#pragma once

#include "common.h"

// ---- bf16 path: MFMA kernels (kernels_bf16.hip) ----
// V^T over the scratch slots of all sequences: slot p (position t of sequence b) holds eta * E[ids[b][t+1]] for
// t < T and a valid id, else 0; K-blocked [S/64][d][64]. Vrow (nullable): the same rows row-major and unscaled,
// [S][d]. cfac (nullable; batch layout only): clipping factors [B][ceil(T/C)]; V^T's position t is also scaled
// by cfac[b][t/C].
hipError_t launch_gather_vt_bf16(const int32_t *ids, const bf16_t *E, int vocab, bf16_t *VT, bf16_t *Vrow,
                                 const float *cfac, float eta, const Layout &lay, hipStream_t s);
// Z = SiLU(x W_gate^T) * (x W_up^T) -> Z column-blocked [f/64][S][64] (bf16 path; S scratch slots in all).
// Wug: 2f rows of d, interleaved in blocks of 32 (32 up rows, then the matching 32 gate rows), held K-blocked
// by 64 columns: [d/64][2f][64].
hipError_t launch_a1_bf16(const bf16_t *x, const bf16_t *Wug, bf16_t *Z, const Layout &lay, hipStream_t s);
// For each sequence (of the batch, or document): D += sum_p Z[p]^T VT[:, p]^T over its slots (Z column-blocked
// [f/64][S][64], as launch_a1_bf16 writes it; VT carries eta; W[a][i] layout; the state is D = W - W0), from
// state_in[state_in index] or zero, into state_out[state_out index];
// snapshot k of a sequence = bf16(W0 + D at its token k*L), with W0 from its bf16 planes W0p [f/8][d][8].
// Snapshots are planes of 8 columns, [groups in all][f/8][d][8]. cus: compute units of the device (a last
// partial round of at most cus/2 tiles runs as half tiles).
hipError_t launch_update_bf16(const bf16_t *Z, const bf16_t *VT, const float *state_in, float *state_out,
                              bf16_t *snap, const bf16_t *W0p, const Layout &lay, int cus, hipStream_t s);
// P[group][t][s] = <Z[gL+t], Z[gL+s]> if s/C < t/C else 0, for t, s < L (eta is in V^T). cus: compute units of
// the device (the tiles run in rounds of one per CU).
hipError_t launch_scores_bf16(const bf16_t *Z, bf16_t *P, const Layout &lay, int cus, hipStream_t s);
// One snapshot [f/8][d][8] = bf16(W0 + D) of fp32 W0 and state D, [d][f] each (no update).
hipError_t launch_state_to_snap_bf16(const float *W0, const float *D, bf16_t *snap, int d, int f, hipStream_t s);
// bf16 [d][f] -> planes [f/8][d][8].
hipError_t launch_to_planes_bf16(const bf16_t *src, bf16_t *dst, int d, int f, hipStream_t s);
// y[b][gL+t] = Z[gL+t] snap[b][g]^T + sum_s P[b][g][t][s] V[gL+s]; y is bf16, or fp32 with y_f32. cus: compute
// units of the device (the tiles run in rounds of one per CU).
hipError_t launch_out_bf16(const bf16_t *Z, const bf16_t *P, const bf16_t *snap, const bf16_t *VT, void *y,
                           int y_f32, const Layout &lay, int cus, hipStream_t s);
// Per-row chunk Gram sums for clipping: rowpart [B][T_pad/256][wspan][256] fp32. V's rows come from
// Vrow [B][T_pad][d] or, with Vrow null, from E [vocab][d] through ids [B][T+1] (vocab*d*2 < 2^31).
// gv: scratch of clip_gram_scratch_bytes(lay, wspan) bytes. cus: compute units of the device (the tiles run in
// rounds of one per CU).
hipError_t launch_chunk_gram_bf16(const bf16_t *Z, const bf16_t *Vrow, const bf16_t *E, const int32_t *ids, int vocab,
                                  float *gv, float *rowpart, int wspan, const Layout &lay, int cus, hipStream_t s);

// ---- fp32 path: FMA kernels (kernels_f32.hip), same buffers and meaning in fp32 ----
hipError_t launch_gather_vt_f32(const int32_t *ids, const float *E, int vocab, float *VT, float *Vrow,
                                const Layout &lay, hipStream_t s);
// Wug: [2][f][d] (W_up then W_gate).
hipError_t launch_a1_f32(const float *x, const float *Wug, float *Z, float *ZT, float eta, int write_zt,
                         const Layout &lay, hipStream_t s);
// state = D = W - W0; snapshots W0 + D ([B][ngroups][d][f]).
hipError_t launch_update_f32(const float *ZT, const float *VT, float *state, float *snap, const float *W0,
                             const Layout &lay, hipStream_t s);
hipError_t launch_scores_f32(const float *Z, float *P, float eta, const Layout &lay, hipStream_t s);
hipError_t launch_out_f32(const float *Z, const float *P, const float *snap, const float *VT, float *y,
                          const Layout &lay, hipStream_t s);

// ---- update clipping (kernels_clip.hip) ----
// t-tiles per s-tile in rowpart (1 on the fp32 path) and chunks per sequence of a call.
int clip_wspan(const Layout &lay, bool bf16);
// bytes of the bf16 Gram kernel's scratch: 256 KB per workgroup of its grid
size_t clip_gram_scratch_bytes(const Layout &lay, int wspan);
int clip_chunks(const Layout &lay);
// fp32 path: rowpart [B][T_pad] (wspan 1).
hipError_t launch_chunk_gram_f32(const float *Z, const float *Vrow, float *rowpart, const Layout &lay, hipStream_t s);
// c[b][i] = min(1, tau / (|eta| sqrt(sum of chunk i's rows of rowpart))).
hipError_t launch_chunk_factors(const float *rowpart, float *cfac, int wspan, float eta, float tau, const Layout &lay,
                                hipStream_t s);
// Scale slot t of V^T by c[b][t / C] (K-blocked bf16 / row-major fp32 layouts).
hipError_t launch_scale_vt_bf16(bf16_t *VT, const float *cfac, const Layout &lay, hipStream_t s);
hipError_t launch_scale_vt_f32(float *VT, const float *cfac, const Layout &lay, hipStream_t s);

// ---- general target Conv1D(X0) W_target (kernels_target.hip; GEMM in kernels_bf16.hip) ----
// U[b][t] = sum_k cw[k] * E[ids[b][t+1+k]] with the chunk-boundary limit; [B][T_pad][d], rows >= T zero.
hipError_t launch_conv_taps_bf16(const int32_t *ids, const bf16_t *E, int vocab, const float *cw, int K, bf16_t *U,
                                 const Layout &lay, hipStream_t s);
hipError_t launch_conv_taps_f32(const int32_t *ids, const float *E, int vocab, const float *cw, int K, float *U,
                                const Layout &lay, hipStream_t s);
// V = U W_target into V^T (K-blocked bf16, as eta * V / row-major [B][d][T_pad] fp32, unscaled) and, if Vrow,
// row-major V (unscaled). bf16 takes W_target^T [d][d]; fp32 takes W_target [d][d]. cus (bf16): compute units
// of the device (the tiles run in rounds of one per CU).
hipError_t launch_target_gemm_bf16(const bf16_t *U, const bf16_t *WtT, bf16_t *VT, bf16_t *Vrow, float eta,
                                   const Layout &lay, int cus, hipStream_t s);
hipError_t launch_target_gemm_f32(const float *U, const float *W, float *VT, float *Vrow, const Layout &lay,
                                  hipStream_t s);
hipError_t launch_transpose_bf16(const bf16_t *src, bf16_t *dst, int n, hipStream_t s);
hipError_t launch_copy_f32(const float *src, float *dst, long long n, hipStream_t s);

// ---- layout helpers (kernels_misc.hip) ----
// Wug (2f rows of d, K-blocked [d/64][2f][64]) from W_up[f][d], W_gate[f][d]: 32-row blocks, up block then gate
// block.
hipError_t launch_interleave_ug_bf16(const bf16_t *Wu, const bf16_t *Wg, bf16_t *Wug, int f, int d, hipStream_t s);
hipError_t launch_bf16_to_f32(const bf16_t *src, float *dst, long long n, hipStream_t s);
// dst[i] = v for i < n (fp32).
hipError_t launch_fill_f32(float *dst, float v, long long n, hipStream_t s);
// out[b][k] = W0[k] + D[b][k] for b < B, k < n (fp32): the weights of B sequences from their states.
hipError_t launch_add_state_f32(const float *W0, const float *D, float *out, int B, long long n, hipStream_t s);
