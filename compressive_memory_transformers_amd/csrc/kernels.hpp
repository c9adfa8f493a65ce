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
  void* Amat;          // [B*Hkv][s_count][d][d], element type (delta rule only)
  float* Bmat;         // [B*Hkv][s_count][d][d]
  int64_t L, seg_len;
  int32_t units;
  int32_t s_begin, s_count;
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
  int64_t L, seg_len;
  int32_t Hq, Hkv;
  int32_t s_begin, s_count;
  int32_t n_qt;        // query tiles per segment
  float scale_log2;    // log2(e) / sqrt(d)
};

// One streaming decode step (decode.hip): the token at row pos of its
// segment, for every (batch, head).
constexpr int kDecodeMaxGroup = 16;   // query heads per KV head
constexpr int kDecodeMaxChunks = 256;  // 64-row cache chunks (seg_len <= 16384)
struct DecodeArgs {
  const void* q;       // [B][Hq][d]
  const void* k;       // [B][Hkv][d]
  const void* v;       // [B][Hkv][d]
  const float* beta;   // [Hq]
  void* k_cache;       // [B][Hkv][seg_len][d]; row pos is written
  void* v_cache;       // [B][Hkv][seg_len][d]
  const float* M;      // [B][Hkv][d][d]: the state before the segment
  const float* z;      // [B][Hkv][d]
  void* out;           // [B][Hq][d]
  float* part;         // [B*Hkv][n_chunks][G][2 + d]: chunk max, weight sum, value sums
  int64_t seg_len;
  int32_t B, Hq, Hkv, G;
  int32_t pos, n_chunks;  // n_chunks = ceil((pos + 1) / 64)
  float scale_log2;       // log2(e) / sqrt(d)
};

// Wave count of the attention workgroup for a segment length: one wave per 32
// query rows, at most four.
int attn_waves(int64_t seg_len);

hipError_t launch_scan(int dtype, int d, int rule, const ScanArgs& a, hipStream_t stream);
hipError_t launch_affine(int dtype, int d, int rule, const AffineArgs& a, hipStream_t stream);
hipError_t launch_attn(int dtype, int d, const AttnArgs& a, int64_t units, hipStream_t stream);
hipError_t launch_decode(int dtype, int d, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_copy_f32(float* dst, const float* src, int64_t n, hipStream_t stream);

}  // namespace infini
