// Launch interface between the host plan (api.hip) and the kernels
// (scan.hip, attn.hip). Host-visible argument structs and launcher
// declarations only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infini {

enum { kRuleLinear = 0, kRuleDelta = 1 };
enum { kF32 = 0, kBF16 = 1 };

// Memory scan over one window of segments [s_begin, s_begin + s_count):
// per (batch, KV head, 32-column slab of M) it walks the window's segments in
// order, writes the state before each segment (the snapshots) and the state
// after the window.
struct ScanArgs {
  const void* k;       // [B][Hkv][L][d]
  const void* v;       // [B][Hkv][L][d]
  const float* M_in;   // [B][Hkv][d][d]
  const float* z_in;   // [B][Hkv][d]
  float* M_out;        // [B][Hkv][d][d]
  float* z_out;        // [B][Hkv][d]
  void* snapM;         // [B*Hkv][s_count][d (value)][d (key)]: M^T before each segment, element type of q
  float* snapZ;        // [B*Hkv][s_count][d]: z before each segment
  int64_t L, seg_len;
  int32_t units;       // B * Hkv
  int32_t s_begin, s_count;
};

// The affine form of the recurrence (affine.hip): column sums, z prefix,
// per-segment A_s = -Phi^T diag(1/den) Phi and B_s = Phi^T V in parallel, then
// a short sequential chain over the window's segments.
struct AffineArgs {
  const void* k;       // [B][Hkv][L][d]
  const void* v;       // [B][Hkv][L][d]
  const float* M_in;   // [B][Hkv][d][d]
  const float* z_in;   // [B][Hkv][d]
  float* M_out;        // [B][Hkv][d][d]
  float* z_out;        // [B][Hkv][d]
  void* snapM;         // as ScanArgs::snapM
  float* snapZ;        // as ScanArgs::snapZ
  float* colsum;       // [B*Hkv][s_count][d]
  const float* colsum_w;  // products with column sums only: per-row weights of the
                          // sums ([rows of k], laid out as k's rows), or null
  void* Amat;          // [B*Hkv][s_count][d][d], element type (delta rule only)
  float* Bmat;         // [B*Hkv][s_count][d][d]
  float* Amat_f;       // [B*Hkv][s_count][d][d] A_s in float (launch_affine_a_f32 only)
  int64_t L, seg_len;
  int32_t units;
  int32_t s_begin, s_count;
  int32_t reverse;     // chain only: walk the segments last to first
  int32_t heads;       // products only (launch_affine_products): unit u's rows are
                       // those of heads u * heads .. + heads - 1 of k and v, summed;
                       // 0 or 1 in the recurrence
};

// Local causal attention of every (batch, query head, segment, query tile)
// of a window, with the memory retrieval and the gate fused into its epilogue.
struct AttnArgs {
  const void* q;       // [B][Hq][L][d]
  const void* k;       // [B][Hkv][L][d]
  const void* v;       // [B][Hkv][L][d]
  const float* beta;   // [Hq]
  const void* snapM;   // as ScanArgs::snapM
  const float* snapZ;  // as ScanArgs::snapZ
  void* out;           // [B][Hq][L][d]
  float* lse;          // [B][Hq][L] or null: per query row, log2 of the softmax
                       // denominator of the scaled scores, c m + log2(l)
  int64_t L, seg_len;
  int32_t Hq, Hkv;
  int32_t s_begin, s_count;
  // the snapshot of segment s_begin + sl (sl < s_count) is entry
  // unit * snap_count + snap_first + sl of snapM / snapZ
  int32_t snap_first, snap_count;
  int32_t n_qt;        // query tiles per segment
  float scale_log2;    // log2(e) / sqrt(d)
};

// The whole forward in one pass (fused.hip) for bf16, d in {64, 128},
// Hq == Hkv and segments no longer than d: one workgroup per (batch, head)
// walks the segments with the state resident on the chip.
struct FusedArgs {
  const void* q;       // [B][H][L][d]
  const void* k;
  const void* v;
  const float* beta;   // [H]
  const float* M_in;   // [B][H][d][d]
  const float* z_in;   // [B][H][d]
  float* M_out;        // may be M_in
  float* z_out;        // may be z_in
  void* out;           // [B][H][L][d]
  float* lse;          // [B][H][L] or null (as AttnArgs::lse)
  int64_t L;
  int32_t seg_len;     // <= d
  int32_t H;
  int32_t units;       // B * H
  float scale_log2;    // log2(e) / sqrt(d)
};
bool fused_supported(int dtype, int d, int64_t seg_len, int64_t Hq, int64_t Hkv);
hipError_t launch_fused(int d, int rule, const FusedArgs& a, hipStream_t stream);

// One streaming decode step (decode.hip): the token at row pos of its
// segment, for every (batch, head).
constexpr int kDecodeMaxGroup = 16;   // query heads per KV head
constexpr int kDecodeMaxChunks = 256;  // 64-row cache chunks (seg_len <= 16384)
// dk: the key width, dv: the value width (both d for launch_decode).
struct DecodeArgs {
  const void* q;       // [B][Hq][dk]
  const void* k;       // [B][Hkv][dk]
  const void* v;       // [B][Hkv][dv]
  const float* beta;   // [Hq]
  void* k_cache;       // [B][Hkv][seg_len][dk]; row pos is written
  void* v_cache;       // [B][Hkv][seg_len][dv]; row pos is written
  const float* M;      // [B][Hkv][dk][dv]: the state before the segment
  const float* z;      // [B][Hkv][dk]
  void* out;           // [B][Hq][dv]
  float* part;         // [B*Hkv][n_chunks][G][2 + dv]: chunk max, weight sum, value sums
  float* retr;         // [B*Hkv][G][dv]: sigma(q) M of the group's heads
  float* rden;         // [B*Hkv][G]: sigma(q) . z
  int64_t seg_len;
  int32_t B, Hq, Hkv, G;
  int32_t pos, n_chunks;  // n_chunks = ceil((pos + 1) / 64)
  float scale_log2;       // log2(e) / sqrt(dk)
};

// ---- backward pass (bwd.hip) ------------------------------------------------

// Batched matrix product C = alpha op(A) op(B) (+ C if accumulate) with float
// accumulation; A, B in the element type (optionally sigma applied to A as it
// is read), C float. Batch n = hi * S + lo; each operand's offset is
// (hi / div) * stride_hi + lo * stride_lo elements. clip = 1 (2): M (K) is
// the row count of segment lo, min(seg_len, L - lo * seg_len).
struct GemmArgs {
  const void* A;
  const void* B;
  float* C;
  int32_t M, N, K;
  int32_t lda, ldb, ldc;  // row strides as stored: A is M x K (K x M if ta),
                          // B is K x N (N x K if tb), C is M x N
  int32_t ta, tb, a_sigma, accumulate, clip;
  float alpha;
  int32_t batches, S;
  int32_t a_div, b_div, c_div;
  int64_t a_hi, a_lo, b_hi, b_lo, c_hi, c_lo;
  int64_t L, seg_len;
  // epi = 1: C = (alpha op(A) op(B) + w[m] z[n]) sigma'(x[m][n]), with w (float)
  // offset like C's rows (w_hi, w_lo per hi, lo; one value per row), z (float)
  // offset (hi / z_div) z_hi + lo z_lo, x (element type) offset like C.
  int32_t epi, z_div;
  const float* epi_w;
  const float* epi_z;
  const void* epi_x;
  int64_t w_hi, w_lo, z_hi, z_lo;
};

// Everything the backward's elementwise, reduction and attention kernels read.
// Row tensors are [B][H][L] (query heads for q-side, KV heads for k-side).
struct BwdArgs {
  const void* q;       // [B][Hq][L][d]
  const void* k;       // [B][Hkv][L][d]
  const void* v;       // [B][Hkv][L][d]
  const float* beta;   // [Hq]
  const void* out;     // [B][Hq][L][d] forward output
  const float* lse;    // [B][Hq][L] from the training forward
  const void* dout;    // [B][Hq][L][d]
  const void* snapM;   // [B*Hkv][S][d][d] M_{s-1}^T, element type
  const float* snapZ;  // [B*Hkv][S][d] z_{s-1}
  const void* dMsnap;  // [B*Hkv][S][d][d] dM_s^T (dL/dM_s, transposed), element type
  float* nm;           // [B][Hq][L][d] sigma(Q) M_{s-1}, then dL/dQ (retrieval part)
  void* dn;            // [B][Hq][L][d] g dout / den, element type
  float* delta;        // [B][Hq][L] dout . out - g dout . A_mem
  float* dg;           // [B][Hq][L] per-row share of dL/dsigmoid(beta)
  float* dden;         // [B][Hq][L] dL/d(sigma(q) . z)
  float* dk_acc;       // [B][Hkv][L][d]
  float* dv_acc;       // [B][Hkv][L][d]
  float* p_buf;        // [B][Hkv][L][d] sigma(K) M_{s-1} (delta)
  float* du_buf;       // [B][Hkv][L][d] sigma(K) dM_s
  float* dphi;         // [B][Hkv][L][d] dL/dsigma(K) from the update
  void* u_el;          // [B][Hkv][L][d] V - prediction (delta), element type
  void* dp_el;         // [B][Hkv][L][d] dL/dP (delta), element type
  float* dc;           // [B][Hkv][L] dL/dc, c = sigma(k) . z_{s-1} (delta)
  float* phi_f;        // [B][Hkv][L][d] sigma(K) in float (delta)
  float* phic_f;       // [B][Hkv][L][d] sigma(K) / c in float (delta)
  float* wsum_part;    // [B*Hkv][S][chunks][d] partial sums of the dz reductions
  float* e_ret;        // [B*Hkv][S][d] retrieval part of dL/dz_{s-1}
  float* e_upd;        // [B*Hkv][S][d] update part of dL/dz_{s-1}
  float* dzs;          // [B*Hkv][S][d] dL/dz_s
  const float* dz_final;  // [B*Hkv][d] or null
  float* dz0;          // [B*Hkv][d]
  void* dq;            // outputs, element type
  void* dk;
  void* dv;
  float* dbeta;        // [Hq]
  float* dbeta_part;   // [Hq][B][ceil(L / kDbetaChunk)] partial sums of dg
  int32_t dv_final;    // the fused update kernel writes dv itself (dv_acc is not read after it)
  int64_t L, seg_len;
  int32_t B, Hq, Hkv, S;
  int32_t rule;
  float scale_log2;    // log2(e) / sqrt(d)
};

// Positions of one dg row that one workgroup of the d(beta) reduction sums.
constexpr int64_t kDbetaChunk = 4096;

hipError_t launch_gemm(int dtype, const GemmArgs& g, hipStream_t stream);
hipError_t launch_fill_f32(float* p, float v, int64_t n, hipStream_t stream);
// The row steps below take the key width d and the value width dv (both in
// {32, 64, 128}); rows of q, k, z, dk_acc, dphi, phi are d wide, rows of v,
// out, dout, dn, dv_acc, du_buf, p_buf, u_el, dp_el dv wide; nm holds
// sigma(q) M (dv wide) until the retrieval row step, then the retrieval part
// of dQ (d wide).
// Row step of the retrieval backward: delta, dg, dn, dden from nm, out, dout.
hipError_t launch_bwd_retrieval_rows(int dtype, int d, int dv, const BwdArgs& a,
                                     hipStream_t stream);
// e[unit][s] = sum over the segment's rows (and query heads if of_q) of w_t sigma(x_t).
hipError_t launch_bwd_row_weighted_sum(int dtype, int d, int dv, const BwdArgs& a, bool of_q,
                                       hipStream_t stream);
// MFMA kernels of the local-attention gradients (attn_bwd.hip): bf16, d in {64, 128},
// at most 64 query heads per KV head.
bool attn_bwd_mfma_supported(int dtype, int d, int group);
hipError_t launch_attn_bwd_mfma(int d, const BwdArgs& a, hipStream_t stream);
// The retrieval's backward in one MFMA kernel (bf16, same support as above):
// delta, dg, dden, dn and nm from q, out, d_out and the snapshots.
hipError_t launch_bwd_retrieval_mfma(int d, const BwdArgs& a, hipStream_t stream);
// The update's backward in one MFMA kernel (bf16, d in {64, 128}): dv_acc +=
// sigma(K) dM_s, dphi = (V - pred or V) dM_s^T (+ dP M_{s-1}^T), dc.
hipError_t launch_bwd_update_mfma(int d, const BwdArgs& a, hipStream_t stream);
// Local-attention gradients: dk_acc, dv_acc (stored) and dq = nm + attention part.
hipError_t launch_bwd_attention(int dtype, int d, int dv, const BwdArgs& a, hipStream_t stream);
// Row step of the delta rule's update backward (after p_buf, du_buf).
hipError_t launch_bwd_update_rows(int dtype, int d, int dv, const BwdArgs& a, hipStream_t stream);
// phi_f = sigma(K), phic_f = sigma(K) / (sigma(K) . z_{s-1}), per key row, in float.
hipError_t launch_bwd_phi_rows(int dtype, int d, int dv, const BwdArgs& a, hipStream_t stream);
// dst[i] = src[i] rounded to the element type (or copied, float).
hipError_t launch_round_f32(int dtype, void* dst, const float* src, int64_t n, hipStream_t stream);
// dz suffix scan and the final dK, dV, dbeta.
hipError_t launch_bwd_finish(int dtype, int d, int dv, const BwdArgs& a, hipStream_t stream);

// Wave count of the attention workgroup for a segment length: one wave per 32
// query rows, at most four.
int attn_waves(int64_t seg_len);

hipError_t launch_scan(int dtype, int d, int rule, const ScanArgs& a, hipStream_t stream);
// The direct scan with d_key = dk != d_value = dv (both in {32, 64, 128}): M is
// [dk][dv] per unit, the snapshots M^T [dv][dk], z [dk].
hipError_t launch_scan_kv(int dtype, int dk, int dv, int rule, const ScanArgs& a,
                          hipStream_t stream);
hipError_t launch_affine(int dtype, int d, int rule, const AffineArgs& a, hipStream_t stream);
// A_s = -Phi^T diag(1/den) Phi in float into a.Amat_f, for every (unit,
// segment) of a.s_count, from K (bf16, d = 128) and the z before each segment
// (a.snapZ): the delta rule's transition as the backward's state gradient needs it.
bool affine_a_f32_supported(int dtype, int d);
hipError_t launch_affine_a_f32(const AffineArgs& a, hipStream_t stream);
// The chain step of the affine form alone (a.reverse honoured).
hipError_t launch_chain(int dtype, int d, int rule, const AffineArgs& a, hipStream_t stream);
// The same step in float with d_key = dk != d_value = dv: M, B_s [dk][dv] per
// (unit, segment), A_s [dk][dk], snapshots M^T [dv][dk].
hipError_t launch_chain_kv_f32(int dk, int dv, int rule, const AffineArgs& a,
                               hipStream_t stream);
// The linear rule's products alone, Bmat = sum over a.heads heads of
// sigma(K)^T V per (unit, segment), bf16 with d = 128 (hipErrorInvalidValue
// otherwise: the caller takes another path). With a.colsum set, also the
// column sums of sigma(K) over the same rows, weighted by a.colsum_w when
// that is set.
hipError_t launch_affine_products(int dtype, int d, const AffineArgs& a, hipStream_t stream);
hipError_t launch_attn(int dtype, int d, const AttnArgs& a, int64_t units, hipStream_t stream);
// The attention with d_key = dk != d_value = dv: q, k rows of dk, v and out
// rows of dv, snapshots as launch_scan_kv writes them.
hipError_t launch_attn_kv(int dtype, int dk, int dv, const AttnArgs& a, int64_t units,
                          hipStream_t stream);
hipError_t launch_decode(int dtype, int d, const DecodeArgs& a, hipStream_t stream);
// The decode step with d_key = dk and d_value = dv (each 32, 64 or 128): q, k
// and the key cache rows of dk, v, the value cache rows and out of dv, M [dk][dv].
hipError_t launch_decode_kv(int dtype, int dk, int dv, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t stream);
// One snapshot per unit from a state: snapM[u] = M[u]^T ([dv][dk], element
// type), snapZ[u] = z[u]; M [units][dk][dv], z [units][dk] float.
hipError_t launch_snapshot(int dtype, int dk, int dv, const float* M, const float* z,
                           void* snapM, float* snapZ, int64_t units, hipStream_t stream);

// The projections around the block (proj.hip): C[m][n] = sum_k A[m][k] W[n][k]
// in bf16 with float accumulation, W [N][K] row-major. A is read as rows
// (a_mode kProjRows: A[m][k] = a[m lda + k]) or gathered from a head-major
// [B][Ha][L][d] tensor (kProjGather: A[b L + t][h d + j] = a[((b Ha + h) L + t)
// d + j]); C is written as rows (kProjRows: c[m ldc + n]) or split into heads
// (kProjHeads: column h d + j goes to q, k or v [b][h][t][j], the Hq query
// heads first, then Hkv key heads, then Hkv value heads). Requires K % 32 == 0,
// N % 4 == 0 and, for a gathered A, d % 32 == 0.
constexpr int kProjRows = 0, kProjGather = 1, kProjHeads = 1;
struct ProjArgs {
  const void* a;  // bf16 throughout
  const void* w;
  void* c;
  void* q;
  void* k;
  void* v;
  int64_t M, N, K;
  int64_t lda, ldc;
  int64_t a_elems;  // elements of the tensor a points into (bounds of its loads)
  int64_t L, d, Ha, Hq, Hkv;  // d: the gathered A's head width; heads of q and k (kProjHeads)
  int64_t dv;                  // heads of v (kProjHeads)
  int32_t a_mode, c_mode;
};
hipError_t launch_proj(const ProjArgs& a, hipStream_t stream);

}  // namespace infini
