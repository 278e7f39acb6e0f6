// Grouped expert GEMMs with one workgroup per CU and the weights streamed
// straight into registers: the prefill gate/up for balanced bf16 layers (and
// their down GEMM, with the weights in fragment order), and both GEMMs (bf16,
// fp8 or MXFP4 weights) at a few dozen rows per expert.
//
// Same arithmetic as the other expert kernels (each expert a SwiGLU MLP,
// Reflection Beam 1.0 overview, section "Mixture of Experts"; the SwiGLU
// product in FP32, section "Residual stream"):
//   h = bf16( SiLU(x Wg^T) * (x Wu^T) )      gate/up
//   y = bf16( h Wd^T )                        down
// FP8 (OCP e4m3) weights convert exactly to bf16 in registers; the
// per-output-channel scale multiplies the fp32 accumulator in the epilogue.
// MXFP4 weights (E2M1 codes, one E8M0 scale per 32 inputs) convert with their
// block scale to bf16 in registers, exactly.
//
// A workgroup takes one row tile of an expert (MT blocks of 16 rows) and a
// block of output columns.  What sets the streaming rate of a CU is the bytes
// it keeps in flight; here:
//
//   * 8 waves (two per SIMD); every wave spans all the tile's rows and owns
//     NB column blocks of 16 (gate/up: NB/2 gate blocks and the matching up
//     blocks).  No other wave needs its weight rows.
//   * Each wave's weight rows go HBM -> VGPRs with 16-byte buffer loads into
//     a ring of four 64-k windows, three ahead of the MFMAs.
//   * The activation rows (x, gathered through the permutation, or the
//     expert's h rows), needed by every wave, go HBM/L2 -> LDS with
//     direct-to-LDS buffer loads into a ring of four stages, also three
//     windows ahead.  One load instruction covers 8 rows x one row's whole
//     128-byte window slice, lane l taking row l/8 and 16-byte chunk
//     (l%8) ^ (l/8) ^ (group%2), so every MFMA operand reads back with one
//     conflict-free ds_read_b128 (the same swizzle as the LDS-tiled kernels).
//     A window's 2*MT groups go round the waves; groups wholly past the
//     tile's rows, and the waves' loads past the last group, read past the
//     buffer's end (zeros, without a memory access) into one spare slot.
//   * Lane (r = l%16, q = l/16) of MFMA half a of a window uses k in
//     [16q + 8a, +8) of the window for both operands (fp8: the lane's 16
//     weight bytes are k [16q, 16q + 16), half a the a-th 8 of them).  With
//     the weights in fragment order (1 KB lane-ordered 64-byte column slices
//     of 16-row blocks) a load instruction reads 8 whole 128-byte lines
//     (bf16: four 256-byte runs; fp8, MXFP4: one 1 KB slice) instead of 16
//     rows x 64 bytes.
//     MXFP4 windows are 128 deep: lane q's 16 code bytes are k [32q, +32),
//     one scale block, and MFMA slice t uses k [32q + 8t, +8); the
//     activations sit as two 64-deep halves, so the lane reads half q/2,
//     chunk 4(q%2) + t (every lane group of a ds_read_b128 shares q, so the
//     swizzle keeps it conflict-free).  A row's scale bytes for the ring's
//     four windows arrive as one 16-byte load with ring slot 0.
//   * Every row block runs every window (rows past the tile's end hold its
//     last row, zeros or stale values, and are never stored: an MFMA output
//     row depends on its own A row only), so the compute has no branches and
//     reads its activation fragments three blocks ahead of their MFMAs.
//   * Each stage is its own LDS array, so the compiler tells a wave's loads
//     into one stage from reads of another and waits for the former only:
//     before the window's barrier every wave reads back a word of each slot
//     it filled in that stage (the compiler waits for those loads), and the
//     barrier then publishes the stage to every wave; it also says every wave
//     is done with the stage (and the registers) the next issue reuses.
//   * That issue (window w+3's loads) goes between the MFMAs of window w,
//     evenly, not in one block after the barrier: there the eight waves'
//     loads queued at the CU's address unit at once, and a wave could start
//     its MFMAs only once its last load had been accepted.
//   * The output tile is staged through LDS and stored as whole 16-byte
//     chunks along rows.
//   * Work items (row tile, column block) are dealt to the 8 XCDs in
//     contiguous ranges, so the workgroups of one expert share its
//     activation rows in one L2.
//
// Balanced bf16 GEMMs (272-row tiles, NB = 2).  A window brings 34 KB of
// activation rows (L2 hits) per 32 KB of weights (HBM) through each CU's
// vector memory path.  With row-order weights its address unit was about 71%
// busy and set the time (MFMAs 53% of the cycles); with fragment-order weights
// it is about 55% busy, the MFMAs about 60%, and the chip holds its power
// limit at about 1.7 GHz.
// At 96-row tiles (NB = 4) the work is HBM-bound: a window brings 12 KB of
// activations and 64 KB (bf16) of weights per CU.
#include <type_traits>
#include <utility>

#include "common.h"

namespace beam {

constexpr int kWWin = 64;                    // k per window: one 128-byte line of a bf16 row
constexpr int kWAhead = 3;                   // windows in flight ahead of the one multiplied
constexpr int kWRing = kWAhead + 1;          // LDS stages = weight register buffers
constexpr int kWWaves = 8;
constexpr int kWXcds = 8;
constexpr int kWBalancedMT = 17;             // 272-row tiles: a whole balanced expert
constexpr int kWModerateMT = 6;              // 96-row tiles: up to 64 rows per expert on average
constexpr int kWDenseTileGroup = 4;          // dense layers: row tiles per group of the work order

enum { kWGateUp = 0, kWDown = 1 };
enum { kWtBF16 = 0, kWtFP8 = 1, kWtMX = 2 };

template <int WT, int MODE, int MT, int NB>
struct WideCfg {
  static constexpr int WIN_K = WT == kWtMX ? 128 : 64;         // k per window
  static constexpr int HALVES = WIN_K / 64;                   // 64-deep activation halves per window
  static constexpr int WIN_BYTES = WT == kWtBF16 ? 128 : 64;  // weight bytes per row per window
  static constexpr int ROWS = 16 * MT;
  static constexpr int GROUPS = 2 * MT;                       // 8-row activation load groups per window
  static constexpr int GPW = (GROUPS + kWWaves - 1) / kWWaves;
  static constexpr int WLD = WT == kWtBF16 ? 2 : 1;           // 16-byte weight loads per block per window
  static constexpr int COLS = MODE == kWGateUp ? kWWaves * 8 * NB : kWWaves * 16 * NB;   // output columns
  static constexpr int CST = COLS * 2 + 16;                   // staged output row stride, bytes
  static constexpr int OUT_ROWS = (ROWS + kWRing - 1) / kWRing;   // output rows staged per stage
  static constexpr int SUB = (GROUPS + 1) * 1024;             // a 64-deep half + one spare slot
  static constexpr int A_BYTES = HALVES * SUB;
  static constexpr int STAGE = ((A_BYTES > OUT_ROWS * CST ? A_BYTES : OUT_ROWS * CST) + 1023) / 1024 * 1024;
  static_assert(kWRing * STAGE <= 160 * 1024, "LDS");
  static_assert(MODE == kWDown || NB % 2 == 0, "gate/up blocks come in pairs");
};

typedef __attribute__((address_space(3))) void wlds_void;

constexpr int kRsrcWord3 = 0x00020000;       // raw buffer resource, 32-bit data format
constexpr uint32_t kPastEnd = 0x80000000u;   // a buffer offset past every resource's extent (< 2^31)

// A stage's direct-to-LDS loads (a plain device function: the host pass of a kernel template drops
// an instantiation that names this builtin in a lambda).
__device__ __forceinline__ void stage_fill(uint8_t* st, __amdgpu_buffer_rsrc_t rsrc, const int* slot,
                                           const uint32_t* off, int n, int soff) {
#pragma unroll
  for (int i = 0; i < n; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (wlds_void*)(st + slot[i]), 16, off[i], soff, 0, 0);
}

// Scheduling groups of one window's compute: NI times (NB MFMAs, one DS read, and the i-th share of NV
// vector memory loads, spread evenly).
template <int N>
__device__ __forceinline__ void vmem_group() {
  if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(0x010, N, 0);
}
template <int NB, int NV, int NI, int... Is>
__device__ __forceinline__ void mfma_read_load_groups(std::integer_sequence<int, Is...>) {
  ((__builtin_amdgcn_sched_group_barrier(0x008, NB, 0), __builtin_amdgcn_sched_group_barrier(0x100, 1, 0),
    vmem_group<(Is + 1) * NV / NI - Is * NV / NI>()),
   ...);
}

// Row-block counts compiled per tile height: a tile of n row blocks runs the smallest count >= n.
// 272-row tiles: skewed routing leaves many experts a tile of one or two blocks (the balanced
// layer's experts take 16 or 17); 96-row tiles: three to six blocks at 64 rows per expert.  (Some
// larger sets, e.g. with 12 added, make the compiler spill registers in the 272-row down kernel.)
template <int... Vs>
struct RowBlockSet {
  template <typename F>
  __device__ static void dispatch(int nmb, F&& f) {
    bool done = false;
    ((done || nmb > Vs ? void() : (f(std::integral_constant<int, Vs>{}), void(done = true))), ...);
  }
};
template <int MT>
struct WideRowBlocks;
template <>
struct WideRowBlocks<17> : RowBlockSet<1, 2, 4, 8, 16, 17> {};
template <>
struct WideRowBlocks<6> : RowBlockSet<2, 3, 4, 5, 6> {};

// (The weight pointers are not restrict: with them the compiler moves each window's weight loads
// down to their first use, three windows later, which empties the pipeline.)
template <int WT, int MODE, int MT, int NB>
__global__ __launch_bounds__(512) void wide_kernel(int H, int I, int K, const uint16_t* __restrict__ act,
                                                   const void* w0, const void* w1, const void* s0, const void* s1,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ sorted_pairs,
                                                   const int32_t* __restrict__ tiles,
                                                   const int32_t* __restrict__ ntiles, uint16_t* __restrict__ out,
                                                   long act_bytes, int tgroup, int packed) {
  using C = WideCfg<WT, MODE, MT, NB>;
  constexpr bool FP8 = WT == kWtFP8, MX = WT == kWtMX;
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds2[C::STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t lds3[C::STAGE];
  auto stage = [&](auto sc) -> uint8_t* {
    constexpr int S = decltype(sc)::value;
    if constexpr (S == 0) return lds0;
    else if constexpr (S == 1) return lds1;
    else if constexpr (S == 2) return lds2;
    else return lds3;
  };

  const int KD = MODE == kWGateUp ? H : I;                  // reduction length
  const int NT = (MODE == kWGateUp ? I : H) / C::COLS;      // column blocks per tile
  // Work items in groups of tgroup row tiles, column block outer and tile inner within a group (the
  // last group padded; tgroup = 1: one tile's column blocks after another).  tgroup = 0: the row
  // tiles of one expert form the group (the tile list holds an expert's tiles in a row, tile k of
  // the expert at rows k * ROWS), so an expert with several tiles streams each weight column block
  // for all of them at once, and one-tile experts keep the tile order.
  const int nitems = tgroup == 0 ? ntiles[0] * NT : (ntiles[0] + tgroup - 1) / tgroup * tgroup * NT;
  const int per_xcd = (nitems + kWXcds - 1) / kWXcds;
  const int slot = blockIdx.x / kWXcds;
  if (slot >= per_xcd) return;
  const int item = (blockIdx.x % kWXcds) * per_xcd + slot;
  if (item >= nitems) return;
  int tile, jn;
  if (tgroup == 0) {
    // the expert's items span the same range as in tile order: the tile there names the expert
    const int tp = item / NT;
    const int ep = tiles[2 * tp];
    const int tfirst = tp - tiles[2 * tp + 1] / C::ROWS;                       // the expert's first tile
    const int ne = (offsets[ep + 1] - offsets[ep] + C::ROWS - 1) / C::ROWS;     // and its tile count
    const int local = item - NT * tfirst;
    jn = local / ne;
    tile = tfirst + local % ne;
  } else {
    const int grp = item / (tgroup * NT), rr = item % (tgroup * NT);
    tile = grp * tgroup + rr % tgroup;
    jn = rr / tgroup;
  }
  if (tile >= ntiles[0]) return;
  const int e = tiles[2 * tile], r0 = tiles[2 * tile + 1];
  const int lo = offsets[e];
  const int rows = min(offsets[e + 1] - lo - r0, C::ROWS);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const int l16 = lane % 16, q = lane / 16;

  // The tile's row blocks pick one of a few compiled row-block counts MTE <= MT: the loop then runs
  // the MFMAs, activation loads and LDS reads of those blocks only (the LDS layout stays MT's).
  auto body = [&](auto mte) {
    constexpr int MTE = decltype(mte)::value;
    constexpr int GROUPS_E = 2 * MTE;                        // 8-row activation load groups per window
    constexpr int GPW = (GROUPS_E + kWWaves - 1) / kWWaves;
    // Activation load groups of this wave: g = wave + 8i, rows 8g + lane/8 (clamped to the tile), as
    // byte offsets into a buffer resource over the activation rows (gate/up: all of x, below 2^31
    // bytes, checked by the launcher; down: the tile's own rows of h).  Loads of groups past the last
    // or wholly past the tile's rows go past the buffer's end, into the spare slot.
    const uint16_t* abase = MODE == kWGateUp ? act : act + (size_t)(lo + r0) * KD;
    const uint32_t abytes = MODE == kWGateUp ? (uint32_t)act_bytes : (uint32_t)rows * KD * 2;
    const __amdgpu_buffer_rsrc_t arsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(abase), (short)0, (int)abytes, kRsrcWord3);
    uint32_t aoff[GPW];
    int aslot[GPW];
  #pragma unroll
    for (int i = 0; i < GPW; ++i) {
      const int gw = wave + kWWaves * i;
      const bool live = gw < GROUPS_E && 8 * gw < rows;
      const int g = gw < GROUPS_E ? gw : GROUPS_E;
      aslot[i] = g * 1024;
      const int r = min(8 * g + lane / 8, rows - 1);
      const uint32_t row = MODE == kWGateUp ? (uint32_t)(sorted_pairs[lo + r0 + r] / K) : (uint32_t)r;
      aoff[i] = live ? (row * (uint32_t)KD + ((lane % 8) ^ (lane / 8) ^ (g % 2)) * 8) * 2 : kPastEnd;
    }
    // This wave's weight rows through buffer resources over the expert's matrices: gate/up, rows
    // c, c + 16, ... of both matrices (c the wave's first intermediate column); down, NB consecutive
    // blocks of 16 rows.  Block n is 16n rows past the first (soffset).
    const int rowb = KD / C::WIN_K * C::WIN_BYTES;                          // bytes per weight row
    const size_t wmat = (size_t)(MODE == kWGateUp ? I : H) * rowb;          // bytes per expert matrix
    const __amdgpu_buffer_rsrc_t wr0 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(w0) + e * wmat), (short)0, (int)wmat, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t wr1 =
        MODE == kWGateUp ? __builtin_amdgcn_make_buffer_rsrc(
                               const_cast<uint8_t*>(static_cast<const uint8_t*>(w1) + e * wmat), (short)0, (int)wmat,
                               kRsrcWord3)
                         : wr0;
    constexpr int WCOLS = MODE == kWGateUp ? 8 * NB : 16 * NB;   // this wave's output columns
    const int wc0 = jn * C::COLS + wave * WCOLS;
    // The lane's 16 bytes of a window.  Row order: row wc0 + l16, bf16 bytes [32q + 16a, +16) of the window
    // (half a), fp8 and MXFP4 bytes [16q, +16).  Fragment order (a window is one 1 KB slice per 64 bytes of
    // row, chunk c of row r at 16(r + 16c)): bf16 slice q/2, chunk 2(q%2) + a; fp8, MXFP4 chunk q.
    const uint32_t woff = packed ? (uint32_t)wc0 * rowb + (WT == kWtBF16 ? (q / 2) * 1024 + (q % 2) * 512 + l16 * 16
                                                                         : lane * 16)
                                 : (uint32_t)(wc0 + l16) * rowb + q * (C::WIN_BYTES / 4);
    const int wwin = packed ? 16 * C::WIN_BYTES : C::WIN_BYTES;   // bytes between windows
    const int whalf = packed ? 256 : 16;                          // bytes between a bf16 window's two loads
    const int bstride = 16 * rowb;         // bytes between blocks of 16 weight rows
    // where lane (r, q) finds chunk 2q + a of row r of a 16-row block (two 1 KB groups)
    // (MXFP4: chunk 4(q%2) + t of the lane's half q/2, t = 0..3)
    constexpr int NSL = MX ? 4 : 2;   // MFMA slices per window
    int roff[NSL];
  #pragma unroll
    for (int t = 0; t < NSL; ++t) {
      const int c = MX ? 4 * (q % 2) + t : 2 * q + t;
      roff[t] = (MX ? (q / 2) * C::SUB : 0) + (l16 / 8) * 1024 + ((l16 % 8) * 8 + (c ^ (l16 % 8) ^ (l16 / 8))) * 16;
    }
    // MXFP4 scales: KD/32 bytes per weight row; a window's four blocks are one dword (the lane's block
    // is byte q), a round of the ring's four windows one 16-byte load.  Each row's scale bytes are read
    // once per round, not once per window: with a line's worth of rows per workgroup in flight, lines
    // fetched for one window do not reliably stay cached until the next.  In fragment order a round's
    // 16 bytes of the 16 rows of a block are one 256-byte slice (row r at 16r), two whole lines.
    const int srowb = KD / 32;
    const size_t smat = (size_t)(MODE == kWGateUp ? I : H) * srowb;
    const __amdgpu_buffer_rsrc_t sr0 =
        MX ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(static_cast<const uint8_t*>(s0) + e * smat),
                                               (short)0, (int)smat, kRsrcWord3)
           : wr0;
    const __amdgpu_buffer_rsrc_t sr1 =
        MX && MODE == kWGateUp
            ? __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(static_cast<const uint8_t*>(s1) + e * smat),
                                                (short)0, (int)smat, kRsrcWord3)
            : sr0;
    const uint32_t soff = packed ? (uint32_t)wc0 * srowb + l16 * 16 : (uint32_t)(wc0 + l16) * srowb;
    const int sround = packed ? 256 : 16;   // bytes between rounds' scale pieces

    // Stage accesses name the stage arrays themselves: the compiler gives each LDS variable its own
    // alias scope, which lets it match a read of a stage to the direct-to-LDS loads into that stage (and
    // not to loads into the others) when it places its waits.
    // one word of each of this wave's slots in a stage: the compiler waits for all of the wave's loads into it
    auto stage_probe = [&](const uint8_t* st) -> uint32_t {
      uint32_t v = 0;
  #pragma unroll
      for (int h = 0; h < C::HALVES; ++h)
  #pragma unroll
        for (int i = 0; i < GPW; ++i) v |= *reinterpret_cast<const uint32_t*>(st + h * C::SUB + aslot[i] + lane * 16);
      return v;
    };

    u32x4 wb[kWRing][C::WLD][NB];   // [slot][16-byte load][block]; gate/up blocks: NB/2 gate then NB/2 up
    u32x4 wsc[MX ? NB : 1];    // MXFP4 scale dwords of a round's four windows (loaded with ring slot 0)
    u32x4 wsck[MX ? NB : 1];   // the same, kept through the round while the next round's are in flight
    f32x4 acc[MTE][NB];
  #pragma unroll
    for (int m = 0; m < MTE; ++m)
  #pragma unroll
      for (int n = 0; n < NB; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nwin = KD / C::WIN_K;   // a multiple of kWRing (checked by the launcher)
    // Window win into ring slot S.  Past the end the last window is issued again (into a slot nothing
    // reads): every round issues the same loads.
    // (fenced: the direct-to-LDS loads are kept ahead of the weight loads by a scheduling barrier, as the
    // prologue needs; the loop's issues instead leave the placement to compute's scheduling groups)
    auto issue = [&](auto sc, int win, auto fenced) {
      constexpr int S = decltype(sc)::value;
  #pragma unroll
      for (int h = 0; h < C::HALVES; ++h)
        stage_fill(stage(sc) + h * C::SUB, arsrc, aslot, aoff, GPW, (win * C::HALVES + h) * kWWin * 2);
      if constexpr (decltype(fenced)::value) __builtin_amdgcn_sched_barrier(0);   // a fixed load order
      constexpr int NW0 = MODE == kWGateUp ? NB / 2 : NB;   // blocks from the first matrix
      if constexpr (MX && S == 0) {   // window win is a round's first (or, past the end, the last window)
        const int rsoff = sround * (win / kWRing);
  #pragma unroll
        for (int n = 0; n < NW0; ++n)
          wsc[n] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr0, soff, rsoff + n * 16 * srowb, 0));
  #pragma unroll
        for (int n = NW0; n < NB; ++n)
          wsc[n] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(sr1, soff, rsoff + (n - NW0) * 16 * srowb, 0));
      }
      const int wsoff = win * wwin;
  #pragma unroll
      for (int j = 0; j < C::WLD; ++j) {
  #pragma unroll
        for (int n = 0; n < NW0; ++n)
          wb[S][j][n] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr0, woff, wsoff + whalf * j + n * bstride, 0));
  #pragma unroll
        for (int n = NW0; n < NB; ++n)
          wb[S][j][n] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr1, woff, wsoff + whalf * j + (n - NW0) * bstride, 0));
      }
    };
    auto compute = [&](auto sc) {
      constexpr int S = decltype(sc)::value;
      const uint8_t* st = stage(sc);
      float msc[MX ? NB : 1];
      if constexpr (MX) {
  #pragma unroll
        for (int n = 0; n < NB; ++n) {
          if constexpr (S == 0) wsck[n] = wsc[n];   // the next issue into slot 0 reloads wsc
          msc[n] = e8m0_to_f32((wsck[n][S] >> (8 * q)) & 0xFFu);
        }
      }
  #pragma unroll
      for (int a = 0; a < NSL; ++a) {
        bf16x8 b[NB];
  #pragma unroll
        for (int n = 0; n < NB; ++n) {
          if constexpr (MX) {
            b[n] = e2m1x8_to_bf16x8(wb[S][0][n][a], msc[n]);
          } else if constexpr (FP8) {
            const u32x4 v = wb[S][0][n];
            b[n] = e4m3x8_to_bf16x8(a == 0 ? u32x2{v[0], v[1]} : u32x2{v[2], v[3]});
          } else {
            b[n] = __builtin_bit_cast(bf16x8, wb[S][a][n]);
          }
        }
  #pragma unroll
        for (int m = 0; m < MTE; ++m) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(st + m * 2048 + roff[a]);
  #pragma unroll
          for (int n = 0; n < NB; ++n) acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[n], acc[m][n], 0, 0, 0);
        }
      }
      // The next issue's loads (NV of them, issued in this region) go evenly between the MFMA groups: issued
      // all at once after the barrier, a window's loads from the eight waves queue at the CU's address
      // unit, and a wave waiting to issue its last load cannot start its MFMAs.
      constexpr int kAhead = MTE < 3 ? MTE : 3;
      constexpr int kReads = NSL * MTE;
      constexpr int NI = kReads - kAhead;
      constexpr int NV = GPW * C::HALVES + C::WLD * NB + (MX && S == (kWRing - kWAhead) % kWRing ? NB : 0);
      __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);   // DS reads
      mfma_read_load_groups<NB, NV, NI>(std::make_integer_sequence<int, NI>{});
      __builtin_amdgcn_sched_group_barrier(0x008, NB * kAhead, 0);
    };
    // Open the window in ring slot S: this wave's loads into stage S have landed (reading back a word of
    // each slot makes the compiler wait for them), then the barrier: every wave's have, and every wave
    // is done with the window before, whose stage and registers the next issue reuses.
    auto open = [&](auto sc) {
      const uint32_t probe = stage_probe(stage(sc));
      asm volatile("" ::"v"(probe) : "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    // Window w's MFMAs, with window w+3's loads issued among them (into the stage and registers every
    // wave was done with at the barrier).
    auto run = [&](auto sc, int w) {
      constexpr int S = decltype(sc)::value;
      issue(std::integral_constant<int, (S + kWAhead) % kWRing>{}, min(w + kWAhead, nwin - 1), std::false_type{});
      compute(sc);
      __builtin_amdgcn_sched_barrier(0);
    };

    // Each round enters with windows w .. w+2 in flight, issued in the same order on both paths into
    // the loop (prologue and back edge), so the compiler's view of the pending loads at the loop's head
    // is exact and its waits stay precise.
    issue(std::integral_constant<int, 0>{}, 0, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    issue(std::integral_constant<int, 1>{}, 1, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    issue(std::integral_constant<int, 2>{}, 2, std::true_type{});
    __builtin_amdgcn_sched_barrier(0);
    for (int w = 0; w < nwin; w += kWRing) {
      open(std::integral_constant<int, 0>{});
      run(std::integral_constant<int, 0>{}, w);
      open(std::integral_constant<int, 1>{});
      run(std::integral_constant<int, 1>{}, w + 1);
      open(std::integral_constant<int, 2>{});
      run(std::integral_constant<int, 2>{}, w + 2);
      open(std::integral_constant<int, 3>{});
      run(std::integral_constant<int, 3>{}, w + 3);
    }

    // Epilogue: C[r][c] sits in lane (c = l%16, r = 4q + i) of each 16x16 block.  Stage the bf16 output
    // tile row-major in LDS, rows [OUT_ROWS*j, +OUT_ROWS) in stage j (after the repeated tail loads
    // into stages 0..2 have landed and every wave is past the last window), then store whole rows.
    {
      uint32_t probe = 0;
      probe |= stage_probe(lds0);
      probe |= stage_probe(lds1);
      probe |= stage_probe(lds2);
      asm volatile("" ::"v"(probe) : "memory");
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    auto orow = [&](int r) -> uint8_t* {
      const int j = r / C::OUT_ROWS, rr = r % C::OUT_ROWS;
      uint8_t* b = j == 0 ? lds0 : j == 1 ? lds1 : j == 2 ? lds2 : lds3;
      return b + rr * C::CST;
    };
    const int nmb = (rows + 15) / 16;
    if constexpr (MODE == kWGateUp) {
  #pragma unroll
      for (int n = 0; n < NB / 2; ++n) {
        const int c = wave * WCOLS + n * 16 + l16;   // column within the tile
        const float sg = FP8 ? static_cast<const float*>(s0)[(size_t)e * I + jn * C::COLS + c] : 1.f;
        const float su = FP8 ? static_cast<const float*>(s1)[(size_t)e * I + jn * C::COLS + c] : 1.f;
  #pragma unroll
        for (int m = 0; m < MTE; ++m) {
          if (m < nmb) {
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = m * 16 + q * 4 + i;
              const float g = acc[m][n][i] * sg, u = acc[m][n + NB / 2][i] * su;
              *reinterpret_cast<uint16_t*>(orow(r) + c * 2) = f32_to_bf16(silu(g) * u);
            }
          }
        }
      }
    } else {
  #pragma unroll
      for (int n = 0; n < NB; ++n) {
        const int c = wave * WCOLS + n * 16 + l16;
        const float sd = FP8 ? static_cast<const float*>(s0)[(size_t)e * H + jn * C::COLS + c] : 1.f;
  #pragma unroll
        for (int m = 0; m < MTE; ++m) {
          if (m < nmb) {
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = m * 16 + q * 4 + i;
              *reinterpret_cast<uint16_t*>(orow(r) + c * 2) = f32_to_bf16(acc[m][n][i] * sd);
            }
          }
        }
      }
    }
    __syncthreads();
    constexpr int CPR = C::COLS / 8;   // 16-byte chunks per output row
    const int ldo = MODE == kWGateUp ? I : H;
    uint16_t* const obase = out + (size_t)(lo + r0) * ldo + (size_t)jn * C::COLS;
    for (int idx = threadIdx.x; idx < rows * CPR; idx += kWWaves * kWave) {
      const int r = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<u32x4*>(obase + (size_t)r * ldo + ch * 8) = *reinterpret_cast<const u32x4*>(orow(r) + ch * 16);
    }
  };
  WideRowBlocks<MT>::dispatch((rows + 15) / 16, body);
}

// Which one-workgroup-per-CU schedule, if any, a layer takes:
//   * balanced bf16 (more than 64 rows per expert on average with the weights in fragment order,
//     at least 192 in row order, or a dense layer on the LDS-tiled path): the gate/up GEMM, 272-row
//     tiles, each running only the row blocks it holds (with fragment order, against the LDS-tiled
//     kernel: uniform routing at 66, 100 and 134 rows per expert 3.74 / 3.82 / 3.96 against
//     3.86 / 3.97 / 4.29 ms, skewed routing at 94 rows 4.04 against 4.54); the down GEMM too with
//     the weights in fragment order (whole-line weight loads: 1.89 against 2.11 ms on the LDS-tiled
//     kernel at the balanced prefill), else it stays on the LDS-tiled kernel over the same tiles;
//   * MoE layers with 32 to 64 rows per expert on average (bf16, fp8 or MXFP4): both GEMMs, 96-row
//     tiles (a dense layer's single expert would give too few work items).
// The reductions must be whole rounds of the window ring, the column blocks must divide I and H,
// and the token rows and each expert's weight matrix must fit one buffer resource (byte offsets
// below 2^31).
static int wide_mode(const Shape& s, int T) {
  const long tk = (long)T * s.K;
  if (tk < 32L * s.E) return kWideNone;
  if ((long)T * s.H * 2 >= (1L << 31)) return kWideNone;
  if ((long)s.H * s.I * 2 >= (1L << 31)) return kWideNone;   // bf16 bytes bound fp8 and MXFP4 too
  const int wk = s.mx ? 128 : kWWin;   // k per window
  if (s.H % (wk * kWRing) != 0 || s.I % (wk * kWRing) != 0) return kWideNone;
  if (tk <= 64L * s.E)
    return !s.dense && s.I % WideCfg<kWtBF16, kWGateUp, kWModerateMT, 4>::COLS == 0 &&
                   s.H % WideCfg<kWtBF16, kWDown, kWModerateMT, 4>::COLS == 0
               ? kWideModerate
               : kWideNone;
  if (!s.fp8 && !s.mx && tk >= (s.packed ? 64L : 192L) * s.E && s.I % WideCfg<kWtBF16, kWGateUp, kWBalancedMT, 2>::COLS == 0 &&
      use_tiled(s, T))
    return kWideBalanced;
  return kWideNone;
}

int wide_schedule(const Shape& s, int T) { return wide_mode(s, T); }

int wide_tile_rows(const Shape& s, int T) {
  return wide_mode(s, T) == kWideBalanced ? 16 * kWBalancedMT : 16 * kWModerateMT;
}

template <int WT, int MODE, int MT, int NB>
static hipError_t wide_launch(const Shape& s, int T, const uint16_t* act, const void* w0, const void* w1,
                              const void* s0, const void* s1, const int32_t* offsets, const int32_t* sorted_pairs,
                              const int32_t* tiles, const int32_t* ntiles, int max_tiles, uint16_t* out,
                              hipStream_t stream) {
  using C = WideCfg<WT, MODE, MT, NB>;
  // a dense layer's row tiles all use the same weights: groups of them run each column block together;
  // at 272-row tiles an expert's own tiles do (skewed routing: 4.55 -> 4.35 ms; one-tile experts
  // unchanged)
  const int tg = s.dense ? kWDenseTileGroup : (MT == kWBalancedMT ? 0 : 1);
  const int tgr = tg ? tg : 1;
  const long items = (long)((max_tiles + tgr - 1) / tgr * tgr) * ((MODE == kWGateUp ? s.I : s.H) / C::COLS);
  const int grid = (int)((items + kWXcds - 1) / kWXcds * kWXcds);
  hipLaunchKernelGGL((wide_kernel<WT, MODE, MT, NB>), dim3(grid), dim3(kWWaves * kWave), 0, stream, s.H, s.I, s.K,
                     act, w0, w1, s0, s1, offsets, sorted_pairs, tiles, ntiles, out, (long)T * s.H * 2, tg,
                     s.packed);
  return hipGetLastError();
}

hipError_t launch_gateup_wide(const Shape& s, int T, const uint16_t* x, const void* wg, const void* wu,
                              const void* sg, const void* su, const int32_t* offsets, const int32_t* sorted_pairs,
                              const int32_t* tiles, const int32_t* ntiles, int max_tiles, uint16_t* h,
                              hipStream_t stream) {
  switch (wide_mode(s, T)) {
    case kWideBalanced:
      return wide_launch<kWtBF16, kWGateUp, kWBalancedMT, 2>(s, T, x, wg, wu, sg, su, offsets, sorted_pairs, tiles,
                                                             ntiles, max_tiles, h, stream);
    case kWideModerate:
      if (s.mx)
        return wide_launch<kWtMX, kWGateUp, kWModerateMT, 4>(s, T, x, wg, wu, sg, su, offsets, sorted_pairs, tiles,
                                                             ntiles, max_tiles, h, stream);
      if (s.fp8)
        return wide_launch<kWtFP8, kWGateUp, kWModerateMT, 4>(s, T, x, wg, wu, sg, su, offsets, sorted_pairs, tiles,
                                                              ntiles, max_tiles, h, stream);
      return wide_launch<kWtBF16, kWGateUp, kWModerateMT, 4>(s, T, x, wg, wu, sg, su, offsets, sorted_pairs, tiles,
                                                             ntiles, max_tiles, h, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_down_wide(const Shape& s, int T, const uint16_t* h, const void* wd, const void* sd,
                            const int32_t* offsets, const int32_t* tiles, const int32_t* ntiles, int max_tiles,
                            uint16_t* y, hipStream_t stream) {
  if (wide_mode(s, T) == kWideBalanced && s.packed)
    return wide_launch<kWtBF16, kWDown, kWBalancedMT, 2>(s, T, h, wd, nullptr, sd, nullptr, offsets, nullptr, tiles,
                                                         ntiles, max_tiles, y, stream);
  if (wide_mode(s, T) != kWideModerate) return hipErrorInvalidValue;
  if (s.mx)
    return wide_launch<kWtMX, kWDown, kWModerateMT, 4>(s, T, h, wd, nullptr, sd, nullptr, offsets, nullptr, tiles,
                                                       ntiles, max_tiles, y, stream);
  if (s.fp8)
    return wide_launch<kWtFP8, kWDown, kWModerateMT, 4>(s, T, h, wd, nullptr, sd, nullptr, offsets, nullptr, tiles,
                                                        ntiles, max_tiles, y, stream);
  return wide_launch<kWtBF16, kWDown, kWModerateMT, 4>(s, T, h, wd, nullptr, sd, nullptr, offsets, nullptr, tiles,
                                                       ntiles, max_tiles, y, stream);
}

}  // namespace beam
