// Shared device helpers and launcher declarations for the Beam MoE kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

namespace beam {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kChunk = 64;        // tokens per permutation chunk (one wave, one bit per token)
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;

// Layer shape as the kernels see it.
struct Shape {
  int H, I, E, G, Gk, K;
  float alpha;
  int fp8;
  int dense = 0;   // one expert holding every token (a dense SwiGLU MLP): no router, no combine
  int mx = 0;      // MXFP4 weights (E2M1 codes + E8M0 block scales); fp8 is 0 then
  int packed = 0;  // weights (and MXFP4 scales) in fragment order: 16-row blocks of lane-ordered slices
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// 8 e4m3 codes (two dwords) -> 8 bf16 values, exact (every e4m3 value is a bf16 value).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(u32x2 q) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 8 E2M1 codes (one dword, element 2i in the low nibble of byte i) times a
// power-of-two block scale -> 8 bf16 values, exact (v_cvt_scalef32_pk_bf16_fp4;
// results assembled through 32-bit casts).
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16x8(uint32_t q, float scale) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 3));
  return __builtin_bit_cast(bf16x8, r);
}

// E8M0 block scale byte -> float 2^(e-127) (codes 1..254; 0 gives 2^-127)
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return __uint_as_float(e ? (e << 23) : 0x00400000u);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// ---- workspace carve-up (host) ----
struct Layout {
  size_t logits, ids, w, masks, counts, offsets, tiles, ntiles, sorted, p2r, h, y, xn, total;
  int ks;        // router k-split
  int nchunks;   // permutation chunks of kChunk tokens
  int max_tiles; // grouped-GEMM row tiles
};

// ---- launchers (host; each enqueues on `stream`, returns hipError_t of the launch) ----
hipError_t launch_router_logits(const Shape& s, int T, int ks, const uint16_t* x, const float* wr,
                                float* partial, hipStream_t stream);
hipError_t launch_router_select(const Shape& s, int T, int ks, const float* partial, const float* b,
                                int32_t* ids, float* w, hipStream_t stream);
hipError_t launch_permute(const Shape& s, int T, const int32_t* ids, int nchunks, uint64_t* masks,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_to_row,
                          int tile_rows, int32_t* tiles, int32_t* ntiles, hipStream_t stream);
hipError_t launch_gateup(const Shape& s, int T, const uint16_t* x, const void* wg, const void* wu,
                         const void* sg, const void* su, const int32_t* offsets, const int32_t* sorted_pairs,
                         const int32_t* tiles, const int32_t* ntiles, int max_tiles, int kparts, float* part,
                         uint16_t* h, hipStream_t stream);
hipError_t launch_down(const Shape& s, int T, const uint16_t* h, const void* wd, const void* sd,
                       const int32_t* offsets, const int32_t* tiles, const int32_t* ntiles, int max_tiles,
                       int kparts, float* part,
                       uint16_t* y, hipStream_t stream);
hipError_t launch_combine(const Shape& s, int T, const uint16_t* y, const float* w,
                          const int32_t* pair_to_row, uint16_t* out, hipStream_t stream);
int down_kparts(const Shape& s, int T);
int gateup_kparts(const Shape& s, int T);
hipError_t launch_pack_fragments(long rows, int row_bytes, int slice_bytes, const void* src, void* dst,
                                 hipStream_t stream);
hipError_t launch_mxfp4_quantize(int rows, int cols, const uint16_t* w, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream);
hipError_t launch_dense_setup(int T, int tile_rows, int32_t* offsets, int32_t* sorted_pairs, int32_t* tiles,
                              int32_t* ntiles, hipStream_t stream);
hipError_t launch_rms_norm(int T, int H, float eps, const uint16_t* in, const float* gamma, uint16_t* out,
                           hipStream_t stream);
hipError_t launch_combine_norm_mix(const Shape& s, int T, const uint16_t* y, const float* w, const int32_t* pair_to_row,
                                   float eps, const float* gamma, float a, float b, const uint16_t* stream_in,
                                   uint16_t* stream_out, uint16_t* moe_out, hipStream_t stream);

// Rows per grouped-GEMM tile used for the forward's tile list.
int expert_tile_rows(const Shape& s, int T);

// LDS-tiled expert GEMMs (large token counts): whether T selects them, their tile rows, launchers.
bool use_tiled(const Shape& s, int T);
int tiled_tile_rows();
hipError_t launch_gateup_tiled(const Shape& s, const uint16_t* x, const void* wg, const void* wu, const float* sg,
                               const float* su, const int32_t* offsets, const int32_t* sorted_pairs,
                               const int32_t* tiles, const int32_t* ntiles, int max_tiles, int tile_rows, uint16_t* h,
                               hipStream_t stream);
hipError_t launch_down_tiled(const Shape& s, const uint16_t* h, const void* wd, const float* sd,
                             const int32_t* offsets, const int32_t* tiles, const int32_t* ntiles, int max_tiles,
                             int tile_rows, uint16_t* y, hipStream_t stream);

// Expert GEMMs with one workgroup per CU and the weights streamed into registers: which schedule T
// selects (the balanced one runs gate/up, and down too with the weights in fragment order), its tile
// rows, launchers.
enum { kWideNone = 0, kWideBalanced = 1, kWideModerate = 2 };
int wide_schedule(const Shape& s, int T);
int wide_tile_rows(const Shape& s, int T);
hipError_t launch_gateup_wide(const Shape& s, int T, const uint16_t* x, const void* wg, const void* wu,
                              const void* sg, const void* su, const int32_t* offsets, const int32_t* sorted_pairs,
                              const int32_t* tiles, const int32_t* ntiles, int max_tiles, uint16_t* h,
                              hipStream_t stream);
hipError_t launch_down_wide(const Shape& s, int T, const uint16_t* h, const void* wd, const void* sd,
                            const int32_t* offsets, const int32_t* tiles, const int32_t* ntiles, int max_tiles,
                            uint16_t* y, hipStream_t stream);

}  // namespace beam
