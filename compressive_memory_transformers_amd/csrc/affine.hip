// The memory recurrence in affine form, parallel over segments.
//
// "Infini-Attention" (AI Wiki), "How does the compressive memory work?": per
// segment, with Phi = sigma(K_s) and den_t = Phi_t . z_{s-1},
//   delta:  M_s = M_{s-1} + Phi^T (V_s - Phi M_{s-1} / den)
//              = M_{s-1} + Phi^T V_s - (Phi^T diag(1/den) Phi) M_{s-1}
//   linear: M_s = M_{s-1} + Phi^T V_s
//   both:   z_s = z_{s-1} + sum_t Phi_t.
// Written this way, every product over the segment's N tokens depends on K, V
// and z only, not on M. So the O(N d^2) work runs for all segments at once, and
// only a d x d by d x d product per segment stays sequential:
//   1. colsum:  c_s = sum_t sigma(K_s,t)                 (parallel over segments)
//   2. prefix:  z_{s-1} = z_0 + sum_{s'<s} c_s'           (a short loop over s)
//   3. affine:  A_s = -Phi^T diag(1/den) Phi, B_s = Phi^T V_s   (parallel)
//   4. chain:   M_s = M_{s-1} + B_s + A_s M_{s-1}        (sequential, per slab of M)
// The chain writes the state before each segment (M^T in the element type, as
// the attention kernel's retrieval reads it); step 2 writes z before each
// segment. This pays off when N is large next to d: the sequential part costs
// 2 d^3 per segment instead of the direct scan's 6 N d^2.
//
// Precision: A_s is stored in the element type (its product with M is a small
// correction); B_s and M stay in float. V never passes through a rounding of
// V - prediction, which would lose the prediction.
#include "common.hpp"
#include "kernels.hpp"
#include "lds_tile.hpp"

namespace infini {

namespace {

// ---- 1. column sums of sigma(K) per (unit, segment) ------------------------

template <typename T, int D>
__global__ __launch_bounds__(256) void colsum_kernel(AffineArgs a) {
  constexpr int CG = D / 8;      // 8-column groups of a row
  constexpr int TL = 256 / CG;   // token lanes
  __shared__ float red[TL * D];
  const int tid = threadIdx.x, cg = tid % CG, tl = tid / CG;
  const int unit = blockIdx.x / a.s_count, sl = blockIdx.x % a.s_count;
  const int64_t seg_start = (int64_t)(a.s_begin + sl) * a.seg_len;
  const int n_s = (int)min<int64_t>(a.seg_len, a.L - seg_start);
  const T* K = static_cast<const T*>(a.k) + ((int64_t)unit * a.L + seg_start) * D + 8 * cg;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // eight rows per step, loaded before any is used, so eight loads are in
  // flight (with one workgroup per segment and two per CU, four left the
  // kernel at about 4.3 TB/s, bound by the bytes in flight)
  constexpr int UR = 8;
  int t = tl;
  for (; t + (UR - 1) * TL < n_s; t += UR * TL) {
    frag_t<T> kv[UR];
#pragma unroll
    for (int u = 0; u < UR; ++u) kv[u] = load8<T>(K + (int64_t)(t + u * TL) * D);
#pragma unroll
    for (int u = 0; u < UR; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += feature_map(to_f32<T>(kv[u][e]));
  }
  for (; t < n_s; t += TL) {
    const frag_t<T> kv = load8<T>(K + (int64_t)t * D);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += feature_map(to_f32<T>(kv[e]));
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[tl * D + 8 * cg + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int j = 0; j < TL; ++j) s += red[j * D + tid];
    a.colsum[((int64_t)unit * a.s_count + sl) * D + tid] = s;
  }
}

// ---- 2. z before each segment, and after the window ------------------------

// The column sums do not depend on z, so their loads run kPrefetch segments
// ahead of the running sum (a ring of registers, the loop unrolled so every
// slot index is a constant); only the additions are sequential.
constexpr int kPrefetch = 16;

template <int D>
__global__ __launch_bounds__(D) void prefix_kernel(AffineArgs a) {
  const int unit = blockIdx.x, tid = threadIdx.x;
  const int n = a.s_count;
  const float* cs = a.colsum + (int64_t)unit * n * D + tid;
  float* sz = a.snapZ + (int64_t)unit * n * D + tid;
  float z = a.z_in[(int64_t)unit * D + tid];
  float ring[kPrefetch];
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) ring[u] = u < n ? cs[(int64_t)u * D] : 0.f;
  for (int s0 = 0; s0 < n; s0 += kPrefetch) {
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u) {
      const int sl = s0 + u;
      if (sl < n) {
        sz[(int64_t)sl * D] = z;
        z += ring[u];
        if (sl + kPrefetch < n) ring[u] = cs[(int64_t)(sl + kPrefetch) * D];
      }
    }
  }
  a.z_out[(int64_t)unit * D + tid] = z;
}

// ---- 3. A_s = -Phi^T diag(1/den) Phi and B_s = Phi^T V_s --------------------

template <int D, int RULE>
struct AffineShape {
  static constexpr int RT = D / 32;                                // row tiles (key dim)
  static constexpr int CT = (RULE == kRuleDelta ? 2 : 1) * (D / 32);  // column tiles
  static constexpr int NTILE = RT * CT;
  static constexpr int NW = NTILE < 8 ? NTILE : 8;
  static constexpr int TPW = NTILE / NW;  // tiles per wave
  static_assert(NTILE % NW == 0, "tile split");
};

template <typename T, int D, int RULE>
__global__ __launch_bounds__((AffineShape<D, RULE>::NW * 64)) void affine_kernel(AffineArgs a) {
  using S = AffineShape<D, RULE>;
  constexpr int NW = S::NW, NT = NW * 64, RT = S::RT, TPW = S::TPW;
  constexpr bool DELTA = RULE == kRuleDelta;
  constexpr int TC = 64;                  // tokens per chunk
  constexpr int TS = TC + pad16<T>();     // row stride of the transposed tiles
  constexpr int CG = D / 8;               // 8-column groups
  constexpr int ITEMS = (TC / 4) * CG;    // (4 tokens x 8 columns) staging items
  constexpr int IPT = (ITEMS + NT - 1) / NT;

  __shared__ __align__(16) T PhiT[D * TS];                 // sigma(K)^T  [key dim][token]
  __shared__ __align__(16) T DPhiT[DELTA ? D * TS : 1];    // (Phi / den)^T
  __shared__ __align__(16) T VT[D * TS];                   // V^T         [value dim][token]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 31, h = lane >> 5;
  const int unit = blockIdx.x / a.s_count, sl = blockIdx.x % a.s_count;
  const int64_t seg_start = (int64_t)(a.s_begin + sl) * a.seg_len;
  const int n_s = (int)min<int64_t>(a.seg_len, a.L - seg_start);
  const T* K = static_cast<const T*>(a.k) + ((int64_t)unit * a.L + seg_start) * D;
  const T* V = static_cast<const T*>(a.v) + ((int64_t)unit * a.L + seg_start) * D;
  const float* z = a.snapZ + ((int64_t)unit * a.s_count + sl) * D;

  f32x16 acc[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) acc[j] = zero16();

  // registers of the staging items of the current chunk (kr, vr) and of the
  // next ones (kr1/vr1, kr2/vr2): with 2-byte elements two chunks of loads are
  // in flight while one is staged and multiplied (float elements: one)
  constexpr bool DEEP = sizeof(T) == 2;
  frag_t<T> kr[IPT][4], vr[IPT][4], kr1[IPT][4], vr1[IPT][4], kr2[IPT][4], vr2[IPT][4];
  auto load_chunk = [&](int t0, frag_t<T> (&kx)[IPT][4], frag_t<T> (&vx)[IPT][4]) {
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + it * NT;
      const int cg = item % CG, tq = item / CG;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + 4 * tq + q;
        kx[it][q] = zero_frag<T>();
        vx[it][q] = zero_frag<T>();
        if (item < ITEMS && t < n_s) {
          kx[it][q] = load8<T>(K + (int64_t)t * D + 8 * cg);
          vx[it][q] = load8<T>(V + (int64_t)t * D + 8 * cg);
        }
      }
    }
  };
  float zc[IPT][8];
#pragma unroll
  for (int it = 0; it < IPT; ++it) {
    const int cg = (tid + it * NT) % CG;
#pragma unroll
    for (int e = 0; e < 8; ++e) zc[it][e] = z[8 * cg + e];
  }

  load_chunk(0, kr, vr);
  if (DEEP) load_chunk(TC, kr1, vr1);  // rows past n_s are not loaded (zeros)
  for (int t0 = 0; t0 < n_s; t0 += TC) {
    // stage the chunk: sigma, den, transposed stores
#pragma unroll
    for (int it = 0; it < IPT; ++it) {
      const int item = tid + it * NT;
      const int cg = item % CG, tq = item / CG;
      float ph[4][8], dp[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = t0 + 4 * tq + q < n_s;
        dp[q] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ph[q][e] = ok ? feature_map(to_f32<T>(kr[it][q][e])) : 0.f;
          dp[q] += ph[q][e] * zc[it][e];
        }
      }
      float rd[4];  // 1 / den_t
      if constexpr (DELTA) {
        // den_t: sum over the CG lanes that hold token t's columns
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          dp[q] = row_sum<CG>(dp[q]);
          rd[q] = 1.f / dp[q];
        }
      }
      if (item < ITEMS) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          vec4_t<T> p4, v4;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            p4[q] = from_f32<T>(ph[q][e]);
            v4[q] = vr[it][q][e];
          }
          store4<T>(PhiT + (8 * cg + e) * TS + 4 * tq, p4);
          store4<T>(VT + (8 * cg + e) * TS + 4 * tq, v4);
          if constexpr (DELTA) {
            vec4_t<T> d4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const bool ok = t0 + 4 * tq + q < n_s;
              d4[q] = from_f32<T>(ok ? ph[q][e] * rd[q] : 0.f);
            }
            store4<T>(DPhiT + (8 * cg + e) * TS + 4 * tq, d4);
          }
        }
      }
    }
    __syncthreads();
    if (DEEP) {
      if (t0 + 2 * TC < n_s) load_chunk(t0 + 2 * TC, kr2, vr2);  // in flight for two chunks
    } else {
      if (t0 + TC < n_s) load_chunk(t0 + TC, kr1, vr1);  // in flight during the products
    }

#pragma unroll
    for (int kc = 0; kc < TC / 16; ++kc) {
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int tile = w * TPW + j;
        const int rt = tile % RT, ct = tile / RT;
        const frag_t<T> af = load8<T>(PhiT + (32 * rt + i) * TS + 16 * kc + 8 * h);
        const T* bsrc;
        if (DELTA && ct < RT) bsrc = DPhiT + (32 * ct + i) * TS;
        else bsrc = VT + (32 * (ct - (DELTA ? RT : 0)) + i) * TS;
        mma32(acc[j], af, load8<T>(bsrc + 16 * kc + 8 * h));
      }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < IPT; ++it)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        kr[it][q] = kr1[it][q];
        vr[it][q] = vr1[it][q];
        if (DEEP) {
          kr1[it][q] = kr2[it][q];
          vr1[it][q] = vr2[it][q];
        }
      }
  }

  const int64_t base = ((int64_t)unit * a.s_count + sl) * D * D;
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int tile = w * TPW + j;
    const int rt = tile % RT, ct = tile / RT;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * rt + acc_row(r, h);
      if (DELTA && ct < RT)
        static_cast<T*>(a.Amat)[base + (int64_t)row * D + 32 * ct + i] = from_f32<T>(-acc[j][r]);
      else
        a.Bmat[base + (int64_t)row * D + 32 * (ct - (DELTA ? RT : 0)) + i] = acc[j][r];
    }
  }
}

// One 4-byte LDS-DMA load per lane as inline assembly, like dma16_asm (the
// kernel waits for it explicitly): lane l's dword lands at lds + 4 l.
__device__ __forceinline__ void dma4_asm(void* lds, u32x4 rsrc, uint32_t voff) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(m), "v"(voff), "s"(rsrc) : "memory");
}

// ---- 3'. the same products for bf16, d = 128, from DMA-fed LDS tiles ---------
//
// Chunks of 32 tokens of K and V stream into a 3-deep LDS ring (K in the "K"
// layout, V in the "V" layout, lds_tile.hpp). All 512 threads then stage the
// chunk in place, row major: 16 threads per token, 8 columns each, form
// sigma(K) and its dot with z (the 16 partial dots summed by DPP), and write
// Phi and Phi / den in the "V" layout. The products read every operand with
// transposing LDS reads (the token index is the k index): wave w owns the
// 2 x 2 (delta) or 2 x 1 (linear) block of 32 x 32 output tiles at row tiles
// 2 (w / 4), + 1 and column tiles 2 (w % 4), + 1 of [Phi/den | V] (delta), or
// column tile w % 4 of V (linear). The LDS (64 KB) leaves room for two
// workgroups per CU, so one's staging (VALU) runs beside the other's
// products (MFMA).
// COLSUM (linear rule): also the segment's column sums of Phi, from the staged
// rows (the linear rule's products need no z, so the sums need no pass of
// their own over K); with a.colsum_w set, the sums weight each row by it
// (the backward's sum over the group's query rows of dden_t sigma(q_t), beside
// C_s in the same pass over q). The weights of a chunk come into an LDS ring
// by one 4-byte DMA per lane of wave 0, counted in that wave's waits.
template <int RULE, bool COLSUM = false>
__global__ __launch_bounds__(512, 2) void affine_dma_kernel(AffineArgs a) {
  constexpr int D = 128, NW = 8, TC = 32, NBUF = 3;
  constexpr bool DELTA = RULE == kRuleDelta;
  constexpr int BC = DELTA ? 2 : 1;  // column tiles per wave (row tiles: 2)
  using Tile = DmaTile<D, NW, TC>;
  __shared__ __align__(1024) bf16 Kr[NBUF][TC * D];
  __shared__ __align__(1024) bf16 Vr[NBUF][TC * D];
  __shared__ __align__(1024) bf16 Ph[TC * D];
  __shared__ __align__(1024) bf16 DPh[DELTA ? TC * D : 8];
  __shared__ __align__(16) float Zs[256];
  __shared__ __align__(16) float Ws[COLSUM ? NBUF * 64 : 4];  // row weights, a ring

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.x / a.s_count, sl = blockIdx.x % a.s_count;
  const int64_t seg_start = (int64_t)(a.s_begin + sl) * a.seg_len;
  const int n_s = (int)min<int64_t>(a.seg_len, a.L - seg_start);
  const bool weighted = COLSUM && a.colsum_w != nullptr;  // uniform
  // rows of `heads` consecutive heads (one in the recurrence), chunk c of
  // the run being chunk c % n_c of head c / n_c
  const int heads = a.heads > 1 ? a.heads : 1;
  const bf16* K = static_cast<const bf16*>(a.k) + ((int64_t)unit * heads * a.L + seg_start) * D;
  const bf16* V = static_cast<const bf16*>(a.v) + ((int64_t)unit * heads * a.L + seg_start) * D;
  const int n_c = (n_s + TC - 1) / TC;
  const int n_t = heads * n_c;
  auto head_off = [&](int c) { return (int64_t)(c / n_c) * a.L * D; };
  auto chunk0 = [&](int c) { return (c % n_c) * TC; };

  // staging role: token st_t of the chunk, columns 8 st_g .. + 7. z comes
  // into LDS by one 16-byte DMA per lane of wave 0 (lanes past d / 4 read
  // outside the resource, which returns zeros), issued before the tiles, so
  // the first chunk's wait covers it.
  const int st_t = tid >> 4, st_g = tid & 15;
  if (w == 0)
    dma16_asm(Zs, asm_rsrc(a.snapZ + ((int64_t)unit * a.s_count + sl) * D, D * 4),
              (uint32_t)lane * 16, 0u);
  float zc[8];
  Tile tile;
  tile.init(w, lane);
  // chunk c's weights into ring slot c % NBUF (lanes past the chunk's rows
  // read zeros; the slot holds all 64 lanes)
  auto issue_w = [&](int c) {
    if (weighted && w == 0) {
      const int64_t r0 = ((int64_t)unit * heads + c / n_c) * a.L + seg_start + chunk0(c);
      const int rows = min(TC, n_s - chunk0(c));
      dma4_asm(Ws + (c % NBUF) * 64, asm_rsrc(a.colsum_w + r0, (uint32_t)rows * 4),
               (uint32_t)lane * 4);
    }
  };
  tile.template issue_asm<true>(K, Kr[0], 0, n_s, w);
  tile.template issue_asm<false>(V, Vr[0], 0, n_s, w);
  issue_w(0);
  if (n_t > 1) {
    tile.template issue_asm<true>(K + head_off(1), Kr[1], chunk0(1), n_s, w);
    tile.template issue_asm<false>(V + head_off(1), Vr[1], chunk0(1), n_s, w);
    issue_w(1);
  }

  // product role: row tiles rt0, rt0 + 1; column tiles BC cq + c
  const int rt0 = 2 * (w >> 2), cq = w & 3;
  uint32_t ao[2], bo[BC];
#pragma unroll
  for (int r = 0; r < 2; ++r) ao[r] = tr_offset<D>(lane, rt0 + r);
#pragma unroll
  for (int c = 0; c < BC; ++c) bo[c] = tr_offset<D>(lane, (BC * cq + c) & 3);
  f32x16 acc[2][BC];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < BC; ++c) acc[r][c] = zero16();
  float csum[8];  // COLSUM: columns 8 st_g .. + 7 over this thread's token slot
#pragma unroll
  for (int e = 0; e < 8; ++e) csum[e] = 0.f;

  for (int ch = 0; ch < n_t; ++ch) {
    const int buf = ch % NBUF;
    // this wave's loads of chunk ch have landed (the 2 PER_WAVE of chunk
    // ch + 1, issued later, and wave 0's weight load of it may still be in
    // flight)
    if (ch + 1 < n_t) {
      if (weighted && w == 0)
        wait_vmcnt<2 * Tile::PER_WAVE + 1>();
      else
        wait_vmcnt<2 * Tile::PER_WAVE>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();  // chunk ch complete everywhere; chunk ch - 1's products done
    if (ch == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) zc[e] = Zs[8 * st_g + e];
    }
    if (ch + 2 < n_t) {  // into the buffer chunk ch - 1 used
      const int cn = ch + 2;
      tile.template issue_asm<true>(K + head_off(cn), Kr[cn % NBUF], chunk0(cn), n_s, w);
      tile.template issue_asm<false>(V + head_off(cn), Vr[cn % NBUF], chunk0(cn), n_s, w);
      issue_w(cn);
    }
    // stage Phi and Phi / den of token st_t (zero past the segment's end)
    {
      const bool ok = chunk0(ch) + st_t < n_s;
      const float wt = weighted ? Ws[buf * 64 + st_t] : 1.f;
      const bf16x8 kv = load8<bf16>(Kr[buf] + st_t * D + 8 * (st_g ^ swz_k<D>(st_t)));
      float ph[8];
      float dp = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = ok ? feature_map((float)kv[e]) : 0.f;
        ph[e] = f;
        dp += f * zc[e];
        if constexpr (COLSUM) csum[e] += wt * f;
      }
      const int po = st_t * D + 8 * (st_g ^ swz_v<D>(st_t));
      {
        bf16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (bf16)ph[e];
        store8<bf16>(Ph + po, y);
      }
      if constexpr (DELTA) {
        const float den = row_sum<16>(dp);
        const float rd = ok ? 1.f / den : 0.f;
        bf16x8 y;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (bf16)(ph[e] * rd);
        store8<bf16>(DPh + po, y);
      }
    }
    __syncthreads();
    // products over the chunk's TC / 16 k chunks of 16 tokens
#pragma unroll
    for (int p = 0; p < TC / 16; ++p) {
      bf16x8 af[2], bf[BC];
#pragma unroll
      for (int r = 0; r < 2; ++r) af[r] = tr_frag<D>(Ph, ao[r], p);
#pragma unroll
      for (int c = 0; c < BC; ++c) {
        const bool of_v = !DELTA || BC * cq + c >= 4;
        bf[c] = tr_frag<D>(of_v ? Vr[buf] : DPh, bo[c], p);
      }
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int c = 0; c < BC; ++c) mma32(acc[r][c], af[r], bf[c]);
    }
  }

  if constexpr (COLSUM) {
    // sum the TC token slots of each column in LDS (the K ring, contiguous
    // and free now: [TC slots][128 columns] floats, 16 KB over Kr[0], Kr[1])
    static_assert(TC * D * 4 <= 2 * TC * D * 2, "the sums fit in two ring buffers");
    float* red = reinterpret_cast<float*>(&Kr[0][0]);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) red[st_t * D + 8 * st_g + e] = csum[e];
    __syncthreads();
    if (tid < D) {
      float cs = 0.f;
      for (int t = 0; t < TC; ++t) cs += red[t * D + tid];
      a.colsum[((int64_t)unit * a.s_count + sl) * D + tid] = cs;
    }
  }

  const int i = lane & 31, h = lane >> 5;
  const int64_t base = ((int64_t)unit * a.s_count + sl) * D * D;
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < BC; ++c) {
      const int ct = BC * cq + c;  // of [Phi/den | V] (delta) or of V (linear)
      const bool is_a = DELTA && ct < 4;
      const int col = 32 * (ct & 3) + i;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = 32 * (rt0 + r) + acc_row(q, h);
        if (is_a)
          static_cast<bf16*>(a.Amat)[base + (int64_t)row * D + col] = (bf16)(-acc[r][c][q]);
        else
          a.Bmat[base + (int64_t)row * D + col] = acc[r][c][q];
      }
    }
}

// ---- 3''. A_s in float, for the backward's state gradient -------------------
//
// The transition I + A_s of the delta rule has entries of order 1 / z, so the
// state gradient's reversed chain needs A_s = -Phi^T diag(1/den) Phi to about
// float accuracy (one bf16 product leaves each term 2^-8 off). The staging is
// affine_dma_kernel's (chunks of 32 tokens of K through a 3-deep DMA ring,
// 16 threads per token), but Phi and Phi / den are each staged as a pair of
// bf16 values, hi = bf16(x) and lo = bf16(x - hi), and every output tile takes
// three bf16 products per k step: hi^T hi + hi^T lo + lo^T hi, summed in float.
// Each term is then within about 2^-16 of its float value (the split and the
// dropped lo^T lo), and the terms are all positive (Phi > 0, den > 0), so the
// sums do not cancel. Wave w owns the output row tile w / 2 and the column
// tiles 2 (w % 2) and + 1.
__global__ __launch_bounds__(512, 2) void affine_af32_kernel(AffineArgs a) {
  constexpr int D = 128, NW = 8, TC = 32, NBUF = 3;
  using Tile = DmaTile<D, NW, TC>;
  __shared__ __align__(1024) bf16 Kr[NBUF][TC * D];
  __shared__ __align__(1024) bf16 Ph[TC * D];  // Phi, hi and lo parts
  __shared__ __align__(1024) bf16 Pl[TC * D];
  __shared__ __align__(1024) bf16 Qh[TC * D];  // Phi / den, hi and lo parts
  __shared__ __align__(1024) bf16 Ql[TC * D];
  __shared__ __align__(16) float Zs[256];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.x / a.s_count, sl = blockIdx.x % a.s_count;
  const int64_t seg_start = (int64_t)(a.s_begin + sl) * a.seg_len;
  const int n_s = (int)min<int64_t>(a.seg_len, a.L - seg_start);
  const bf16* K = static_cast<const bf16*>(a.k) + ((int64_t)unit * a.L + seg_start) * D;
  const int n_c = (n_s + TC - 1) / TC;

  // staging role: token st_t of the chunk, columns 8 st_g .. + 7; z by one
  // 16-byte DMA per lane of wave 0 (lanes past d / 4 read zeros), issued
  // before the tiles, so the first chunk's wait covers it
  const int st_t = tid >> 4, st_g = tid & 15;
  if (w == 0)
    dma16_asm(Zs, asm_rsrc(a.snapZ + ((int64_t)unit * a.s_count + sl) * D, D * 4),
              (uint32_t)lane * 16, 0u);
  Tile tile;
  tile.init(w, lane);
  tile.template issue_asm<true>(K, Kr[0], 0, n_s, w);
  if (n_c > 1) tile.template issue_asm<true>(K, Kr[1], TC, n_s, w);

  const int rt = w >> 1, c0 = 2 * (w & 1);
  const uint32_t ao = tr_offset<D>(lane, rt);
  const uint32_t bo[2] = {tr_offset<D>(lane, c0), tr_offset<D>(lane, c0 + 1)};
  f32x16 acc[2] = {zero16(), zero16()};
  float zc[8];

  for (int ch = 0; ch < n_c; ++ch) {
    const int buf = ch % NBUF;
    // this wave's load of chunk ch has landed (chunk ch + 1's may be in flight)
    if (ch + 1 < n_c)
      wait_vmcnt<Tile::PER_WAVE>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // chunk ch complete everywhere; chunk ch - 1's products done
    if (ch == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) zc[e] = Zs[8 * st_g + e];
    }
    if (ch + 2 < n_c)  // into the buffer chunk ch - 1 used
      tile.template issue_asm<true>(K, Kr[(ch + 2) % NBUF], (ch + 2) * TC, n_s, w);
    {  // stage the splits of token st_t (zero past the segment's end)
      const bool ok = ch * TC + st_t < n_s;
      const bf16x8 kv = load8<bf16>(Kr[buf] + st_t * D + 8 * (st_g ^ swz_k<D>(st_t)));
      float ph[8];
      float dp = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = ok ? feature_map((float)kv[e]) : 0.f;
        ph[e] = f;
        dp += f * zc[e];
      }
      const float den = row_sum<16>(dp);
      const float rd = ok ? 1.f / den : 0.f;
      bf16x8 h1, l1, h2, l2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        h1[e] = (bf16)ph[e];
        l1[e] = (bf16)(ph[e] - (float)h1[e]);
        const float x = ph[e] * rd;
        h2[e] = (bf16)x;
        l2[e] = (bf16)(x - (float)h2[e]);
      }
      const int po = st_t * D + 8 * (st_g ^ swz_v<D>(st_t));
      store8<bf16>(Ph + po, h1);
      store8<bf16>(Pl + po, l1);
      store8<bf16>(Qh + po, h2);
      store8<bf16>(Ql + po, l2);
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < TC / 16; ++p) {
      const bf16x8 ah = tr_frag<D>(Ph, ao, p), al = tr_frag<D>(Pl, ao, p);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 bh = tr_frag<D>(Qh, bo[c], p), bl = tr_frag<D>(Ql, bo[c], p);
        mma32(acc[c], ah, bh);
        mma32(acc[c], ah, bl);
        mma32(acc[c], al, bh);
      }
    }
  }

  const int i = lane & 31, h = lane >> 5;
  float* A = a.Amat_f + ((int64_t)unit * a.s_count + sl) * D * D;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int col = 32 * (c0 + c) + i;
#pragma unroll
    for (int q = 0; q < 16; ++q) A[(32 * rt + acc_row(q, h)) * D + col] = -acc[c][q];
  }
}

// ---- 4. M_s = M_{s-1} + B_s + A_s M_{s-1}, per 32-column slab ---------------
//
// With a.reverse the same step runs over the segments last to first. The
// backward pass uses it for the gradient of the state: A_s is symmetric
// (-Phi^T diag(1/den) Phi), so dM_{s-1} = dM_s + A_s dM_s + C_s has this form
// with B_s = C_s, and the snapshot written before step s is dM_s.

// D: the rows of M (the key width), DV: its columns (the value width); A_s is
// D x D.
template <typename T, int D, int RULE, int DV = D>
__global__ __launch_bounds__(D / 32 * 64) void chain_kernel(AffineArgs a) {
  constexpr int NC = D / 16;
  constexpr int MTS = D + pad16<T>();
  constexpr bool DELTA = RULE == kRuleDelta;
  __shared__ __align__(16) T Mt[DELTA ? 32 * MTS : 1];  // M_{s-1}^T of the slab

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i = lane & 31, h = lane >> 5;
  const int slab = blockIdx.x % (DV / 32), unit = blockIdx.x / (DV / 32);
  const int col0 = 32 * slab;

  // this lane's 16 entries of the slab: rows 32w + acc_row(r, h), column col0 + i
  f32x16 acc;
  const float* Min = a.M_in + (int64_t)unit * D * DV;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = Min[(32 * w + acc_row(r, h)) * DV + col0 + i];

  // B_s (this lane's 16 entries of the slab) and A_s (row 32 w + i) of step
  // `it`; they do not depend on M, so each step's loads are issued a step
  // ahead (the last step reloads its own, in bounds and unused)
  auto seg_of = [&](int it) {
    return (int64_t)unit * a.s_count + (a.reverse ? a.s_count - 1 - it : it);
  };
  auto load_step = [&](int it, float* bv, frag_t<T>* af) {
    const int64_t seg = seg_of(it);
    const float* Bs = a.Bmat + seg * D * DV;
#pragma unroll
    for (int r = 0; r < 16; ++r) bv[r] = Bs[(32 * w + acc_row(r, h)) * DV + col0 + i];
    if constexpr (DELTA) {
      const T* As = static_cast<const T*>(a.Amat) + seg * D * D + (int64_t)(32 * w + i) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) af[c] = load8<T>(As + 16 * c + 8 * h);
    }
  };
  float bvs[2][16];
  frag_t<T> afs[2][NC];
  if (a.s_count > 0) load_step(0, bvs[0], afs[0]);
  auto step = [&](int it, auto par) {
    constexpr int P = decltype(par)::value;
    load_step(min(it + 1, a.s_count - 1), bvs[P ^ 1], afs[P ^ 1]);
    const float* bv = bvs[P];
    const frag_t<T>* af = afs[P];
    const int64_t seg = seg_of(it);

    // the state before segment s: snapshot (M^T, element type)
    T* sM = static_cast<T*>(a.snapM) + seg * D * DV + (int64_t)(col0 + i) * D + 32 * w + 4 * h;
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      vec4_t<T> y;
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = from_f32<T>(acc[4 * rq + j]);
      store4<T>(sM + 8 * rq, y);
      if constexpr (DELTA) store4<T>(Mt + i * MTS + 32 * w + 8 * rq + 4 * h, y);
    }
    if constexpr (DELTA) {
      __syncthreads();
#pragma unroll
      for (int c = 0; c < NC; ++c) mma32(acc, af[c], load8<T>(Mt + i * MTS + 16 * c + 8 * h));
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += bv[r];
    if constexpr (DELTA) __syncthreads();
  };
  for (int it = 0; it < a.s_count; it += 2) {
    step(it, std::integral_constant<int, 0>{});
    if (it + 1 < a.s_count) step(it + 1, std::integral_constant<int, 1>{});
  }

  float* Mout = a.M_out + (int64_t)unit * D * DV;
#pragma unroll
  for (int r = 0; r < 16; ++r) Mout[(32 * w + acc_row(r, h)) * DV + col0 + i] = acc[r];
}

// ---- the linear rule's chain as a prefix sum over segments -----------------
//
// Under the linear rule M_s = M_{s-1} + B_s: the state before segment s is
// M_0 + sum_{s'<s} B_s', a running sum with no product in it ("Infini-
// Attention" (AI Wiki), "How does the compressive memory work?", the additive
// variant); z is the running sum of the column sums. Every entry is its own
// sum, so the work splits into 32 x 32 blocks of M, one workgroup per (unit,
// block); each walks its unit's segments with the B_s loads kPrefetch
// segments ahead of the additions, and the blocks of column 0 also carry 32
// entries of z. The snapshots (M^T in the element type) go through LDS,
// transposed, four segments per barrier, so both the B_s reads and the
// snapshot writes are whole rows. Same float additions in the same order as
// the step-by-step chain and the z prefix, so the same results.
template <typename T, int D>
__global__ __launch_bounds__(256) void linear_prefix_kernel(AffineArgs a) {
  constexpr int NB = D / 32;  // blocks per side
  constexpr int TS = 32 + 4;  // LDS row stride of a transposed block
  constexpr int GS = 4;       // segments per barrier
  static_assert(kPrefetch % GS == 0, "whole groups per prefetch round");
  __shared__ __align__(16) T Mt[2 * GS][32 * TS];
  const int tid = threadIdx.x;
  const int unit = blockIdx.x / (NB * NB), blk = blockIdx.x % (NB * NB);
  const int r0 = 32 * (blk / NB), c0 = 32 * (blk % NB);
  // float4 of B_s / M: row r0 + rr, columns c0 + 4 cq .. + 3
  const int rr = tid >> 3, cq = tid & 7;
  // snapshot piece: M^T row c0 + tr, rows r0 + 4 tq .. + 3 of M
  const int tr = tid >> 3, tq = tid & 7;
  const int n = a.s_count;
  const int64_t moff = (int64_t)(r0 + rr) * D + c0 + 4 * cq;
  f32x4 acc = *reinterpret_cast<const f32x4*>(a.M_in + (int64_t)unit * D * D + moff);
  const float* Bu = a.Bmat + (int64_t)unit * n * D * D + moff;
  T* snap = static_cast<T*>(a.snapM) + (int64_t)unit * n * D * D +
            (int64_t)(c0 + tr) * D + r0 + 4 * tq;
  // z entries r0 + tid of the unit, in the blocks of column 0 (tid < 32)
  const bool zl = c0 == 0 && tid < 32;
  const int zj = zl ? r0 + tid : 0;
  const float* csu = a.colsum + (int64_t)unit * n * D + zj;
  float* szu = a.snapZ + (int64_t)unit * n * D + zj;
  float z = zl ? a.z_in[(int64_t)unit * D + zj] : 0.f;
  f32x4 ring[kPrefetch];
  float zring[kPrefetch];
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) {
    if (u < n) ring[u] = *reinterpret_cast<const f32x4*>(Bu + (int64_t)u * D * D);
    zring[u] = zl && u < n ? csu[(int64_t)u * D] : 0.f;
  }
  for (int s0 = 0; s0 < n; s0 += kPrefetch) {
#pragma unroll
    for (int g0 = 0; g0 < kPrefetch; g0 += GS) {
      if (s0 + g0 >= n) break;  // uniform
      T (*buf)[32 * TS] = Mt + GS * ((g0 / GS) & 1);
      // the states before the group's segments into LDS, transposed
#pragma unroll
      for (int uu = 0; uu < GS; ++uu) {
        const int u = g0 + uu, sl = s0 + u;
        if (sl < n) {
#pragma unroll
          for (int j = 0; j < 4; ++j) buf[uu][(4 * cq + j) * TS + rr] = from_f32<T>(acc[j]);
          if (zl) szu[(int64_t)sl * D] = z;
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[j] += ring[u][j];
          z += zring[u];
          if (sl + kPrefetch < n) {
            ring[u] = *reinterpret_cast<const f32x4*>(Bu + (int64_t)(sl + kPrefetch) * D * D);
            zring[u] = zl ? csu[(int64_t)(sl + kPrefetch) * D] : 0.f;
          }
        }
      }
      __syncthreads();  // the group's blocks are in LDS (and the other half is free again)
#pragma unroll
      for (int uu = 0; uu < GS; ++uu) {
        const int sl = s0 + g0 + uu;
        if (sl < n) {
          vec4_t<T> y;
#pragma unroll
          for (int j = 0; j < 4; ++j) y[j] = buf[uu][tr * TS + 4 * tq + j];
          store4<T>(snap + (int64_t)sl * D * D, y);
        }
      }
    }
  }
  *reinterpret_cast<f32x4*>(a.M_out + (int64_t)unit * D * D + moff) = acc;
  if (zl) a.z_out[(int64_t)unit * D + zj] = z;
}

// ---- the same step, bf16, d = 128, delta rule: one workgroup per unit ------
//
// The slab kernel above reads A_s whole in each of a unit's four slab
// workgroups, 32 rows per load instruction; with many units that keeps the
// texture units busy for most of its time. Here one 16-wave workgroup holds
// the unit's whole M: wave (rb, cb) owns the 32 x 32 block at rows 32 rb,
// columns 32 cb. Per step A_s comes into LDS once, by 16-byte DMA in the K
// tile layout (two 64-row tiles), M_{s-1}^T is written to LDS in bf16 by the
// waves, and the snapshot goes from there to global memory in 16-byte rows.
// The next step's A_s and B_s block are loaded as soon as the current ones
// are consumed, so their latency overlaps the step's barrier and stores.
// LDS: A_s 32 KiB + M^T 34 KiB; up to 128 registers, one workgroup per CU.
__global__ __launch_bounds__(1024, 4) void chain_unit_kernel(AffineArgs a) {
  constexpr int D = 128, NC = D / 16, MTS = D + 8;
  using Tile = DmaTile<D, 16, 64>;
  __shared__ __align__(1024) bf16 A0[64 * D];  // A_s rows 0..63, K tile layout
  __shared__ __align__(1024) bf16 A1[64 * D];  // rows 64..127
  __shared__ __align__(16) bf16 Mt[D * MTS];   // M_{s-1}^T, [column][row]

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 31, h = lane >> 5;
  const int rb = w >> 2, cb = w & 3;
  const int unit = blockIdx.x;
  const int r0 = 32 * rb, c0 = 32 * cb;

  Tile tile;
  tile.init(w, lane);
  // the A operand: row r0 + i of A_s, k = 16 c + 8 h + e. In the K layout
  // chunk 2c + h of tile row r sits at chunk (2c + h) ^ swz_k(r): byte offset
  // ao ^ 32 c, with ao that of chunk h (the row bits lie above the XOR's).
  const bf16* Ab = rb < 2 ? A0 : A1;
  const uint32_t ao = 2 * (((r0 & 63) + i) * D + 8 * (h ^ swz_k<D>((r0 & 63) + i)));

  f32x16 acc;
  const float* Min = a.M_in + (int64_t)unit * D * D;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = Min[(r0 + acc_row(r, h)) * D + c0 + i];

  const bf16* Amat = static_cast<const bf16*>(a.Amat);
  auto issue_a = [&](int it) {
    const bf16* As = Amat + ((int64_t)unit * a.s_count + it) * D * D;
    tile.template issue<true>(As, A0, 0, 64, w);
    tile.template issue<true>(As + 64 * D, A1, 0, 64, w);
  };
  float bv[16];
  auto load_b = [&](int it) {
    const float* Bs = a.Bmat + ((int64_t)unit * a.s_count + it) * D * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) bv[r] = Bs[(r0 + acc_row(r, h)) * D + c0 + i];
  };
  load_b(0);
  issue_a(0);

  bf16* snap = static_cast<bf16*>(a.snapM);
  for (int it = 0; it < a.s_count; ++it) {
    // M_{s-1}^T of this wave's block into LDS (every wave is past the reads
    // of the previous step: barrier at the loop's end)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      bf16x4 y;
#pragma unroll
      for (int j = 0; j < 4; ++j) y[j] = (bf16)acc[4 * rq + j];
      store4<bf16>(Mt + (c0 + i) * MTS + r0 + 8 * rq + 4 * h, y);
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's part of A_s, and B_s, have landed
    __syncthreads();
    // the snapshot: 16-byte pieces of M^T rows, 32 bytes per thread
    {
      bf16* sM = snap + ((int64_t)unit * a.s_count + it) * D * D;
      const int row = tid >> 3, col = 16 * (tid & 7);
      store8<bf16>(sM + row * D + col, load8<bf16>(Mt + row * MTS + col));
      store8<bf16>(sM + row * D + col + 8, load8<bf16>(Mt + row * MTS + col + 8));
    }
    // M_s = M_{s-1} + A_s M_{s-1} + B_s for this block
#pragma unroll
    for (int c = 0; c < NC; ++c)
      mma32(acc, load8<bf16>(lds_at(Ab, ao ^ (32u * c))),
            load8<bf16>(Mt + (c0 + i) * MTS + 16 * c + 8 * h));
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += bv[r];
    lds_barrier();  // every wave is done with A_s and Mt
    if (it + 1 < a.s_count) {
      issue_a(it + 1);
      load_b(it + 1);
    }
  }

  float* Mout = a.M_out + (int64_t)unit * D * D;
#pragma unroll
  for (int r = 0; r < 16; ++r) Mout[(r0 + acc_row(r, h)) * D + c0 + i] = acc[r];
}

// A_s and B_s (B_s only, linear) of every (unit, segment) of the window.
template <typename T, int D, int RULE>
hipError_t launch_products_t(const AffineArgs& a, hipStream_t stream) {
  const unsigned segs = (unsigned)(a.units * a.s_count);
  if constexpr (sizeof(T) == 2 && D == 128)
    hipLaunchKernelGGL((affine_dma_kernel<RULE>), dim3(segs), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL((affine_kernel<T, D, RULE>), dim3(segs),
                       dim3(AffineShape<D, RULE>::NW * 64), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, int RULE>
hipError_t launch_affine_t(const AffineArgs& a, hipStream_t stream) {
  const unsigned segs = (unsigned)(a.units * a.s_count);
  if constexpr (RULE == kRuleLinear) {
    if (!a.reverse) {
      // the linear rule forward: B_s and the column sums, then both running
      // sums (M and z) in one segment-parallel prefix
      if constexpr (sizeof(T) == 2 && D == 128) {
        // the column sums come out of the products' pass over K
        hipLaunchKernelGGL((affine_dma_kernel<kRuleLinear, true>), dim3(segs), dim3(512), 0,
                           stream, a);
      } else {
        hipLaunchKernelGGL((colsum_kernel<T, D>), dim3(segs), dim3(256), 0, stream, a);
        const hipError_t e = launch_products_t<T, D, RULE>(a, stream);
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL((linear_prefix_kernel<T, D>),
                         dim3((unsigned)(a.units * (D / 32) * (D / 32))), dim3(256), 0, stream, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((colsum_kernel<T, D>), dim3(segs), dim3(256), 0, stream, a);
  hipLaunchKernelGGL((prefix_kernel<D>), dim3((unsigned)a.units), dim3(D), 0, stream, a);
  {
    const hipError_t e = launch_products_t<T, D, RULE>(a, stream);
    if (e != hipSuccess) return e;
  }
  if constexpr (sizeof(T) == 2 && D == 128 && RULE == kRuleDelta) {
    // one workgroup per unit once the units alone fill the CUs; with fewer
    // units the slab kernel's four workgroups per unit keep more CUs busy
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
    if (!a.reverse && a.units >= cus) {
      hipLaunchKernelGGL(chain_unit_kernel, dim3((unsigned)a.units), dim3(1024), 0, stream, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((chain_kernel<T, D, RULE>), dim3((unsigned)(a.units * (D / 32))),
                     dim3(D / 32 * 64), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_affine_rule(int rule, const AffineArgs& a, hipStream_t stream) {
  return rule == kRuleDelta ? launch_affine_t<T, D, kRuleDelta>(a, stream)
                            : launch_affine_t<T, D, kRuleLinear>(a, stream);
}

template <typename T>
hipError_t launch_affine_d(int d, int rule, const AffineArgs& a, hipStream_t stream) {
  switch (d) {
    case 32: return launch_affine_rule<T, 32>(rule, a, stream);
    case 64: return launch_affine_rule<T, 64>(rule, a, stream);
    case 128: return launch_affine_rule<T, 128>(rule, a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename T>
hipError_t launch_chain_d(int d, int rule, const AffineArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.units * (d / 32))), block(d / 32 * 64);
#define INFINI_CHAIN(D)                                                                  \
  if (rule == kRuleDelta)                                                                \
    hipLaunchKernelGGL((chain_kernel<T, D, kRuleDelta>), grid, block, 0, stream, a);     \
  else                                                                                   \
    hipLaunchKernelGGL((chain_kernel<T, D, kRuleLinear>), grid, block, 0, stream, a);
  switch (d) {
    case 32: INFINI_CHAIN(32) break;
    case 64: INFINI_CHAIN(64) break;
    case 128: INFINI_CHAIN(128) break;
    default: return hipErrorInvalidValue;
  }
#undef INFINI_CHAIN
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chain(int dtype, int d, int rule, const AffineArgs& a, hipStream_t stream) {
  return dtype == kBF16 ? launch_chain_d<bf16>(d, rule, a, stream)
                        : launch_chain_d<float>(d, rule, a, stream);
}

template <int DK, int DV>
hipError_t launch_chain_kv_t(int rule, const AffineArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.units * (DV / 32))), block(DK / 32 * 64);
  if (rule == kRuleDelta)
    hipLaunchKernelGGL((chain_kernel<float, DK, kRuleDelta, DV>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((chain_kernel<float, DK, kRuleLinear, DV>), grid, block, 0, stream, a);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_chain_kv_v(int dv, int rule, const AffineArgs& a, hipStream_t stream) {
  switch (dv) {
    case 32: return launch_chain_kv_t<DK, 32>(rule, a, stream);
    case 64: return launch_chain_kv_t<DK, 64>(rule, a, stream);
    case 128: return launch_chain_kv_t<DK, 128>(rule, a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_chain_kv_f32(int dk, int dv, int rule, const AffineArgs& a,
                               hipStream_t stream) {
  switch (dk) {
    case 32: return launch_chain_kv_v<32>(dv, rule, a, stream);
    case 64: return launch_chain_kv_v<64>(dv, rule, a, stream);
    case 128: return launch_chain_kv_v<128>(dv, rule, a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_affine_products(int dtype, int d, const AffineArgs& a, hipStream_t stream) {
  if (dtype != kBF16 || d != 128) return hipErrorInvalidValue;
  const int64_t segs = (int64_t)a.units * a.s_count;
  if (segs > INT32_MAX) return hipErrorInvalidValue;
  if (a.colsum != nullptr)
    hipLaunchKernelGGL((affine_dma_kernel<kRuleLinear, true>), dim3((unsigned)segs), dim3(512), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((affine_dma_kernel<kRuleLinear>), dim3((unsigned)segs), dim3(512), 0,
                       stream, a);
  return hipGetLastError();
}

bool affine_a_f32_supported(int dtype, int d) { return dtype == kBF16 && d == 128; }

hipError_t launch_affine_a_f32(const AffineArgs& a, hipStream_t stream) {
  const int64_t segs = (int64_t)a.units * a.s_count;
  if (segs <= 0 || segs > INT32_MAX || a.Amat_f == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL(affine_af32_kernel, dim3((unsigned)segs), dim3(512), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_affine(int dtype, int d, int rule, const AffineArgs& a, hipStream_t stream) {
  return dtype == kBF16 ? launch_affine_d<bf16>(d, rule, a, stream)
                        : launch_affine_d<float>(d, rule, a, stream);
}

}  // namespace infini
