// The projections around the block: a bf16 GEMM on the matrix cores,
// C[m][n] = sum_k A[m][k] W[n][k], float accumulation.
//
// "Infini-Attention" (AI Wiki), "What happens inside the Infini-attention
// block?": the block forms the query, key and value projections of its input
// tokens, and its gated result goes through the output matrix. Weights are
// stored as a linear layer stores them, (out_features, in_features).
//
// Two ways to read A and two ways to write C, so that neither projection
// needs a layout pass of its own:
//   A rows:    a row-major matrix (the block input x [B L][d_model]);
//   A gather:  the head-major gated result a[b][h][t][j] read as the matrix
//              A[b L + t][h d + j] (the output projection's input);
//   C rows:    a row-major matrix (the block output y);
//   C heads:   column n = h d + j of the fused input projection goes to q,
//              k or v [b][h][t][j] (query heads first, then key, then value).
//
// Tiling. One workgroup of 8 waves computes a 256 x 256 tile of C; wave w
// owns rows 64 (w % 4) .. + 63 and columns 128 (w / 4) .. + 127, as 2 x 4
// MFMA tiles of 32 x 32 (v_mfma_f32_32x32x16_bf16, 128 accumulators a
// lane). The MFMA forms C^T tiles (W rows as the A operand, A rows as the B
// operand), so a lane ends up holding runs of four consecutive columns of one
// row of C: one 8-byte store each.
//
// K advances 32 at a time through a 4-deep LDS ring (A and W slabs of
// 256 x 32, 32 KiB a stage), filled by 16-byte LDS-DMA loads
// (buffer_load ... lds) issued three stages ahead; each wave issues 4 per
// stage. Rows are 64 bytes (four 16-byte chunks); chunk c of row r sits at
// position c ^ ((r >> 2) & 3), so the 16 lanes that one ds_read_b128 cycle
// serves (rows r .. r + 15, one chunk) hit all 64 banks once. The DMA's LDS
// side is fixed (lane i writes bytes 16 i .. 16 i + 15 of its 1 KiB block),
// so the swizzle is applied to the global side: lane i fetches the global
// chunk that belongs at its LDS position.
//
// Tile order: workgroup i runs on XCD i % 8, so consecutive logical tiles are
// dealt out XCD by XCD; within an XCD the tiles come in groups of 8 row
// tiles sweeping the column tiles, so the workgroups resident on one XCD
// share A rows and W rows in its L2.
#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace infini {

namespace {

constexpr int kBM = 256, kBN = 256, kBK = 32, kBuf = 4;
constexpr int kDmaPerWave = 4;  // per stage: 2 for the A slab, 2 for the W slab

// Byte offset, within a 32-row sub-tile, of the fragment lane `lane` reads for
// the k16 step kk (0, 1): row lane % 32, chunk 2 kk + lane / 32, swizzled.
__device__ __forceinline__ uint32_t frag_off(int lane, int kk) {
  const int r = lane & 31;
  const int c = (2 * kk + (lane >> 5)) ^ ((r >> 2) & 3);
  return (uint32_t)(r * kBK * 2 + 16 * c);
}

__device__ __forceinline__ uint32_t rsrc_bytes(int64_t total, int64_t used) {
  const int64_t left = total - used;
  return left <= 0 ? 0u : (left >= (int64_t)0xffffffff ? 0xffffffffu : (uint32_t)left);
}

__global__ __launch_bounds__(512, 1) void proj_kernel(ProjArgs a) {
  __shared__ __align__(1024) bf16 As[kBuf][kBM * kBK];
  __shared__ __align__(1024) bf16 Ws[kBuf][kBN * kBK];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- tile of this workgroup -------------------------------------------------
  const int nM = (int)((a.M + kBM - 1) / kBM), nN = (int)((a.N + kBN - 1) / kBN);
  const int nwg = nM * nN;
  int t = blockIdx.x;
  if (nwg % 8 == 0) t = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  constexpr int kGM = 8;
  const int group = t / (kGM * nN), first = group * kGM;
  const int gsz = min(kGM, nM - first);
  const int within = t - group * kGM * nN;
  const int64_t m0 = (int64_t)(first + within % gsz) * kBM;
  const int64_t n0 = (int64_t)(within / gsz) * kBN;

  // ---- DMA lanes: instruction i of this wave fills rows 16 g .. 16 g + 15,
  // g = 2 w + i, of the A slab (and the same rows of the W slab) ---------------
  const int rr = lane >> 2;
  const int cg = (lane & 3) ^ ((lane >> 4) & 3);  // global chunk of LDS chunk lane & 3
  uint32_t va[2], vw[2];
  const int64_t b0 = m0 / a.L;  // gather: batch element of the tile's first row
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int g = 2 * w + i;
    const int64_t m = min<int64_t>(m0 + 16 * g + rr, a.M - 1);
    if (a.a_mode == kProjGather) {
      const int64_t b = m / a.L, tt = m - b * a.L;
      va[i] = (uint32_t)((((b - b0) * a.Ha * a.L + tt) * a.d + 8 * cg) * 2);
    } else {
      va[i] = (uint32_t)(((m - m0) * a.lda + 8 * cg) * 2);
    }
    const int64_t n = min<int64_t>(n0 + 16 * g + rr, a.N - 1);
    vw[i] = (uint32_t)(((n - n0) * a.K + 8 * cg) * 2);
  }
  const bf16* A = static_cast<const bf16*>(a.a);
  const bf16* W = static_cast<const bf16*>(a.w);
  const int nk = (int)(a.K / kBK);

  // widths are 32, 64 or 128: head and column of an offset by shift and mask
  const int ld = __builtin_ctz((unsigned)a.d);
  const int ldv = __builtin_ctz((unsigned)a.dv);
  // element offsets of the next stage's slabs, advanced stage by stage: a
  // gathered A moves 32 columns within a head, then to the next head's rows
  int64_t a_next = a.a_mode == kProjGather ? b0 * a.Ha * a.L * a.d : m0 * a.lda;
  int64_t w_next = n0 * a.K;
  const int64_t a_jump = a.L * a.d - a.d + kBK;
  int k_next = 0;
  auto issue = [&](int kt) {
    const u32x4 ra = asm_rsrc(A + a_next, rsrc_bytes(a.a_elems * 2, a_next * 2));
    const u32x4 rw = asm_rsrc(W + w_next, rsrc_bytes(a.N * a.K * 2, w_next * 2));
    const int buf = kt & (kBuf - 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = 2 * w + i;
      dma16_asm(&As[buf][16 * g * kBK], ra, va[i], 0u);
      dma16_asm(&Ws[buf][16 * g * kBK], rw, vw[i], 0u);
    }
    k_next += kBK;
    a_next += (a.a_mode == kProjGather && (k_next & (a.d - 1)) == 0) ? a_jump : kBK;
    w_next += kBK;
  };

  // ---- compute lanes ----------------------------------------------------------
  const int wm = w & 3, wn = w >> 2;
  const uint32_t fo0 = frag_off(lane, 0), fo1 = frag_off(lane, 1);
  f32x16 acc[4][2];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) acc[ni][mi] = zero16();

#pragma unroll
  for (int s = 0; s < kBuf - 1; ++s)
    if (s < nk) issue(s);

  for (int kt = 0; kt < nk; ++kt) {
    // this wave's loads of stage kt have landed (later stages may be in flight)
    if (kt + 2 < nk)
      wait_vmcnt<2 * kDmaPerWave>();
    else if (kt + 1 < nk)
      wait_vmcnt<kDmaPerWave>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // stage kt complete everywhere; stage kt - 1's reads done

    // both k16 steps' fragments at once; the first step's products start as
    // soon as its six reads land, and the DMA of stage kt + 3 (into the
    // buffer stage kt - 1 used) goes out between the two steps, its scalar
    // address work overlapping the products in flight. (Timed against a
    // barrier between the two steps with the next stage's reads behind it:
    // this order is faster, the DMA path rather than the barrier being what
    // limits the loop.)
    const int buf = kt & (kBuf - 1);
    const bf16* Ab = &As[buf][(wm * 64) * kBK];
    const bf16* Wb = &Ws[buf][(wn * 128) * kBK];
    bf16x8 xf[2][2], wf[2][4];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint32_t fo = kk ? fo1 : fo0;
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        xf[kk][mi] = load8<bf16>(lds_at(Ab, fo + mi * 32 * kBK * 2));
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
        wf[kk][ni] = load8<bf16>(lds_at(Wb, fo + ni * 32 * kBK * 2));
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) mma32(acc[ni][mi], wf[0][ni], xf[0][mi]);
    if (kt + kBuf - 1 < nk) issue(kt + kBuf - 1);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) mma32(acc[ni][mi], wf[1][ni], xf[1][mi]);
  }

  // ---- epilogue: lane holds C[m][n .. n + 3] for each (ni, mi, quad) -----------
  // (M, N < 2^31 and L < 2^31, checked by the caller: 32-bit row arithmetic)
  const int h = lane >> 5;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int m = (int)m0 + wm * 64 + mi * 32 + (lane & 31);
    if (m >= a.M) continue;
    const unsigned b = (unsigned)m / (unsigned)a.L, tt = (unsigned)m - b * (unsigned)a.L;
    bf16* rowp[3];  // q, k, v at (b, head 0, t, 0); or C's row m
    if (a.c_mode == kProjHeads) {
      rowp[0] = static_cast<bf16*>(a.q) + ((int64_t)b * a.Hq * a.L + tt) * a.d;
      rowp[1] = static_cast<bf16*>(a.k) + ((int64_t)b * a.Hkv * a.L + tt) * a.d;
      rowp[2] = static_cast<bf16*>(a.v) + ((int64_t)b * a.Hkv * a.L + tt) * a.dv;
    } else {
      rowp[0] = rowp[1] = rowp[2] = static_cast<bf16*>(a.c) + (int64_t)m * a.ldc;
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int n = (int)n0 + wn * 128 + ni * 32 + 8 * qd + 4 * h;
        if (n >= a.N) continue;
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (bf16)acc[ni][mi][4 * qd + e];
        bf16* dst;
        if (a.c_mode == kProjHeads) {
          // columns: Hq query heads and Hkv key heads d wide, then Hkv value
          // heads dv wide (four columns never straddle a head: widths are
          // multiples of 32)
          const int nq = (int)a.Hq << ld, nk = nq + ((int)a.Hkv << ld);
          if (n < nk) {
            const int which = n < nq ? 0 : 1, c = n - (which ? nq : 0);
            dst = rowp[which] + (int64_t)(c >> ld) * a.L * a.d + (c & (a.d - 1));
          } else {
            const int c = n - nk;
            dst = rowp[2] + (int64_t)(c >> ldv) * a.L * a.dv + (c & (a.dv - 1));
          }
        } else {
          dst = rowp[0] + n;
        }
        store4<bf16>(dst, v4);
      }
    }
  }
}

}  // namespace

hipError_t launch_proj(const ProjArgs& a, hipStream_t s) {
  const int64_t nM = (a.M + kBM - 1) / kBM, nN = (a.N + kBN - 1) / kBN;
  hipLaunchKernelGGL(proj_kernel, dim3((unsigned)(nM * nN)), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace infini
