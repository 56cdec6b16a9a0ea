// Fused RHT + blockwise absmax 4-bit quantizer and the dequantizer (gfx950).
//
// Method: "Rethinking Shrinkage Bias in LLM FP4 Pretraining" (arXiv
// 2606.20381), paperlayer.ai summary, section 2 ("Blockwise quantization",
// "Rounding rules", "Random Hadamard transforms") and section 4 ("UFP4
// Recipe").  The pages' fused kernel targets other hardware; this is a
// memory-bound design for CDNA4: one block of 16 lives in one lane's
// registers, so the butterfly, absmax and rounding need no cross-lane
// traffic, and loads/stores are laid out so a wave touches contiguous HBM.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "ufp4_device.h"
#include "ufp4_kernels.h"

namespace ufp4 {

// ---------------------------------------------------------------------------
// Row-wise: blocks along the contiguous dimension.  One lane per block of 16;
// consecutive lanes take consecutive blocks of a row, so a wave reads 2 KiB
// and writes 512 B of codes and 256 B of scales contiguously.
//   CONTIG: ld == n_cols == kpad (whole input contiguous, no ragged tail).
//   VEC:    16-byte loads (x 16-byte aligned, ld % 8 == 0), tail guarded.
// ---------------------------------------------------------------------------
template <bool RHT>
__device__ __forceinline__ void unpack16(const uint4 a0, const uint4 a1, uint32_t sign_mask,
                                         float (&v)[16]) {
  const uint32_t w[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = bf16_lo(w[i], RHT ? sign_bit(sign_mask, 2 * i) : 0u);
    v[2 * i + 1] = bf16_hi(w[i], RHT ? sign_bit(sign_mask, 2 * i + 1) : 0u);
  }
}

// Contiguous input (ld == n_cols, n_cols % 16 == 0, 16-byte aligned): block b
// is the 32 bytes at x + 16 b.  A wave owns 64 consecutive blocks (2 KiB) per
// iteration and reads them with two fully coalesced 16-byte-per-lane loads
// (lane l takes bytes 16l and 1024 + 16l); a round trip through LDS then gives
// lane l its own block's 32 bytes.  The grid-stride loop is software
// pipelined: the next chunk's loads are issued before the current chunk is
// processed, and the last prefetch is clamped in range instead of branched.
template <int GRID, int RND, bool RHT>
__device__ __forceinline__ void quantize_store(const uint4 a0, const uint4 a1, int64_t b,
                                               uint8_t *__restrict__ codes,
                                               float *__restrict__ scales, uint32_t sign_mask,
                                               uint32_t seed_lo, uint32_t seed_hi,
                                               uint32_t stream_id) {
  float v[16];
  unpack16<RHT>(a0, a1, sign_mask, v);
  uint32_t w0, w1;
  float s;
  quantize_block<GRID, RND, RHT>(v, (uint64_t)b * 16u, seed_lo, seed_hi, stream_id, w0, w1, s);
  // streaming stores: the outputs are read back only by a later kernel
  __builtin_nontemporal_store(w0, reinterpret_cast<uint32_t *>(codes + b * 8));
  __builtin_nontemporal_store(w1, reinterpret_cast<uint32_t *>(codes + b * 8) + 1);
  __builtin_nontemporal_store(s, scales + b);
}

// Input loads carry the non-temporal hint: every input byte is read exactly
// once, so keeping it in the caches only evicts the outputs being merged
// there (measured at 2^28 elements: row-wise RTNE 123 -> 118 us, column-wise
// 134 -> 129 us, outputs unchanged).  The buffer loads below pass the same
// hint as their cache-policy argument (2).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ntload(const uint4 *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int GRID, int RND, bool RHT>
__global__ __launch_bounds__(256) void quant_rows_contig_kernel(
    const uint16_t *__restrict__ x, int64_t nblk, uint8_t *__restrict__ codes,
    float *__restrict__ scales, uint32_t sign_mask, uint32_t seed_lo, uint32_t seed_hi,
    uint32_t stream_id) {
  __shared__ uint4 s_stage[4][128];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t nfull = nblk / 64;               // chunks of 64 whole blocks
  const int64_t wstride = (int64_t)gridDim.x * 4;
  const int64_t c0 = (int64_t)blockIdx.x * 4 + wave;
  const uint4 *src = reinterpret_cast<const uint4 *>(x);
  uint4 *st = s_stage[wave];
  // Full chunks: no per-lane condition anywhere in the loop, so the compiler's
  // wait counting never has to merge paths and only waits for the loads it
  // needs (one iteration old), never for the stores in flight.
  if (c0 < nfull) {
    uint4 r0 = ntload(src + c0 * 128 + lane), r1 = ntload(src + c0 * 128 + 64 + lane);
    __builtin_amdgcn_s_waitcnt(0);
    for (int64_t c = c0; c < nfull; c += wstride) {
      const int64_t cn = min(c + wstride, nfull - 1);
      const uint4 n0 = ntload(src + cn * 128 + lane), n1 = ntload(src + cn * 128 + 64 + lane);
      st[lane] = r0;
      st[64 + lane] = r1;
      __builtin_amdgcn_wave_barrier();
      const uint4 a0 = st[2 * lane], a1 = st[2 * lane + 1];
      __builtin_amdgcn_wave_barrier();
      quantize_store<GRID, RND, RHT>(a0, a1, c * 64 + lane, codes, scales, sign_mask, seed_lo,
                                     seed_hi, stream_id);
      r0 = n0;
      r1 = n1;
    }
  }
  // The ragged last chunk (fewer than 64 blocks), by one wave.
  if (nblk % 64 != 0 && c0 == nfull % wstride) {
    const int64_t b = nfull * 64 + lane;
    if (b < nblk)
      quantize_store<GRID, RND, RHT>(src[2 * b], src[2 * b + 1], b, codes, scales, sign_mask,
                                     seed_lo, seed_hi, stream_id);
  }
}

// General row-wise input (any stride, alignment or ragged tail): a 2-D
// grid-stride loop over rows and 16-element blocks, so no division is needed;
// VEC rows (16-byte aligned, ld % 8 == 0) use vector loads for full blocks.
template <int GRID, int RND, bool RHT, bool VEC>
__global__ __launch_bounds__(256) void quant_rows_kernel(
    const uint16_t *__restrict__ x, int64_t n_rows, int64_t n_cols, int64_t ld,
    int64_t kblocks, uint8_t *__restrict__ codes, float *__restrict__ scales,
    uint32_t sign_mask, uint32_t seed_lo, uint32_t seed_hi, uint32_t stream_id) {
  for (int64_t row = blockIdx.y; row < n_rows; row += gridDim.y) {
    const uint16_t *xr = x + row * ld;
    for (int64_t kb = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; kb < kblocks;
         kb += (int64_t)gridDim.x * blockDim.x) {
      const int64_t c0 = kb * 16;
      const uint16_t *p = xr + c0;
      float v[16];
      if (VEC && c0 + 16 <= n_cols) {
        unpack16<RHT>(*reinterpret_cast<const uint4 *>(p), *reinterpret_cast<const uint4 *>(p + 8),
                      sign_mask, v);
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t h = (c0 + j < n_cols) ? (uint32_t)p[j] : 0u;
          v[j] = bf16_lo(h, RHT ? sign_bit(sign_mask, j) : 0u);
        }
      }
      const int64_t b = row * kblocks + kb;
      uint32_t w0, w1;
      float s;
      quantize_block<GRID, RND, RHT>(v, (uint64_t)b * 16u, seed_lo, seed_hi, stream_id, w0, w1,
                                     s);
      *reinterpret_cast<uint2 *>(codes + b * 8) = make_uint2(w0, w1);
      scales[b] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Column-wise: blocks along the strided dimension, output transposed.
// A workgroup (4 waves) owns a tile of 256 padded rows (16 blocks) x 64*CW
// columns, CW = 2 or 4 columns per lane (4 for large aligned inputs: each row
// is then read as 512 contiguous bytes per wave, which HBM serves better than
// 256).  Wave w quantizes row-blocks w, w+4, w+8, w+12; in each, lane l loads
// columns CW*l .. CW*l+CW-1 of the 16 rows, and the block's rows come from one
// wave-uniform buffer resource.  The quantized blocks go to LDS and the tile
// is written back as 64*CW output rows of 128 contiguous bytes of codes and 64
// bytes of scales.
// Groups: padded block p belongs to the group e with P_e <= 16p < P_{e+1};
// its rows are off_e + (16p - P_e) + j, zero past the group's end.
// ---------------------------------------------------------------------------
constexpr int kColTileRows = 256;
constexpr int kColTileCols = 128;
constexpr int kMaxGroups = 1024;

__device__ __forceinline__ int64_t clamp_rows(int64_t v, int64_t n) {
  return v < 0 ? 0 : (v > n ? n : v);
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Prefix sums of the groups' padded lengths into LDS (block-wide scan over
// NT threads).
template <int NT = 256>
__device__ __forceinline__ void load_group_tables(const int64_t *__restrict__ goff,
                                                  int n_groups, int64_t n_rows,
                                                  int64_t *s_off, int64_t *s_poff,
                                                  int64_t *s_scan) {
  const int tid = threadIdx.x;
  if (goff == nullptr) {
    if (tid == 0) {
      s_off[0] = 0;
      s_off[1] = n_rows;
      s_poff[0] = 0;
      s_poff[1] = (n_rows + 15) / 16 * 16;
    }
    __syncthreads();
    return;
  }
  // each thread sums the padded counts of a contiguous run of groups
  const int per = (n_groups + NT - 1) / NT;
  const int g0 = tid * per;
  int64_t local = 0;
  // offsets are clamped to [0, n_rows] so that no access leaves the input
  // whatever the device array holds; a decreasing pair is an empty group
  for (int g = g0; g < g0 + per && g < n_groups; ++g) {
    const int64_t a = clamp_rows(goff[g], n_rows), b = clamp_rows(goff[g + 1], n_rows);
    s_off[g] = a;
    local += (b > a) ? (b - a + 15) / 16 * 16 : 0;
  }
  if (tid == 0) s_off[n_groups] = clamp_rows(goff[n_groups], n_rows);
  s_scan[tid] = local;
  __syncthreads();
  // Hillis-Steele inclusive scan over NT partial sums
  for (int d = 1; d < NT; d <<= 1) {
    const int64_t add = tid >= d ? s_scan[tid - d] : 0;
    __syncthreads();
    s_scan[tid] += add;
    __syncthreads();
  }
  int64_t run = tid ? s_scan[tid - 1] : 0;
  for (int g = g0; g < g0 + per && g < n_groups; ++g) {
    s_poff[g] = run;
    const int64_t cnt = s_off[g + 1] - s_off[g];
    run += (cnt > 0) ? (cnt + 15) / 16 * 16 : 0;
  }
  if (tid == NT - 1) s_poff[n_groups] = s_scan[NT - 1];
  __syncthreads();
}

// Largest e with s_poff[e] <= p16 (s_poff non-decreasing, s_poff[0] = 0).
__device__ __forceinline__ int find_group(const int64_t *s_poff, int n_groups, int64_t p16) {
  int lo = 0, hi = n_groups;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_poff[mid] <= p16) lo = mid; else hi = mid;
  }
  return lo;
}

// Raw dwords of one block of 16 rows for this lane's two columns.
template <bool VEC>
__device__ __forceinline__ void load_col_block(const uint16_t *__restrict__ x, int64_t ld,
                                               int64_t n_cols, int64_t row0, int valid,
                                               int col2, uint32_t keep, uint32_t (&w)[16]) {
  // Rows past `valid`, and columns past n_cols in the last valid row, are
  // outside the resource and read as zero; earlier rows' columns past n_cols
  // are masked with `keep`.
  const int64_t nbytes = valid > 0 ? ((int64_t)(valid - 1) * ld + n_cols) * 2 : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(x + row0 * ld), (short)0, (int)nbytes, 0x00020000);
  const int ld2 = (int)(ld * 2);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int off = j * ld2 + col2;
    if (VEC) {
      w[j] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 2) & keep;
    } else {
      const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
      const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs, off + 2, 0, 0);
      w[j] = (lo | (hi << 16)) & keep;
    }
  }
}

// Raw dwords of one block of 16 rows for this lane's CW (2 or 4) columns:
// w[j][c] holds columns 2c, 2c+1 of row j.  With VEC the lane reads CW
// columns with one 4- or 8-byte load per row (rows then need CW-element
// alignment and n_cols a multiple of CW, so a load is wholly in or out of the
// resource); otherwise 2-byte loads.  Out-of-resource reads return zero.
template <bool VEC, int CW>
__device__ __forceinline__ void load_col_rows(const uint16_t *__restrict__ x, int64_t ld,
                                              int64_t n_cols, int64_t row0, int valid,
                                              int colb, const uint32_t (&keep)[CW / 2],
                                              uint32_t (&w)[16][CW / 2]) {
  const int64_t nbytes = valid > 0 ? ((int64_t)(valid - 1) * ld + n_cols) * 2 : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t *>(x + row0 * ld), (short)0, (int)nbytes, 0x00020000);
  const int ld2 = (int)(ld * 2);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int off = j * ld2 + colb;
    if (VEC && CW == 2) {
      w[j][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 2) & keep[0];
    } else if (VEC) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 2);
#pragma unroll
      for (int c = 0; c < CW / 2; ++c) w[j][c] = v[c] & keep[c];
    } else {
#pragma unroll
      for (int c = 0; c < CW / 2; ++c) {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rs, off + 4 * c, 0, 0);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rs, off + 4 * c + 2, 0, 0);
        w[j][c] = (lo | (hi << 16)) & keep[c];
      }
    }
  }
}

// Column-wise tile order.  The tiles of one input (row-band pt, column tile
// ct) are numbered with ORD row bands interleaved (ORD = 1: down a column
// strip first), and the workgroups of each XCD (workgroups are dealt to the 8
// XCDs round robin) take a contiguous range of that numbering, so the tiles an
// XCD runs together write neighbouring pieces of the same output rows and
// those merge in its L2 before they reach HBM.
__device__ __forceinline__ void col_tile_coords(int64_t tile, int64_t n_ptiles, int64_t n_ctiles,
                                                int ord, int64_t &pt, int64_t &ct) {
  const int64_t gsz = (int64_t)ord * n_ctiles;
  const int64_t grp = tile / gsz, r = tile - grp * gsz;
  const int64_t left = n_ptiles - grp * ord;
  const int64_t gb = left < ord ? left : ord;
  pt = grp * ord + r % gb;
  ct = r / gb;
}

// A permutation of the workgroup ids when the grid is a multiple of 8 (the
// launchers make it one), else the identity.
__device__ __forceinline__ int64_t xcd_major_block() {
  if (gridDim.x % 8 != 0) return blockIdx.x;
  return (int64_t)(blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
}

// Stacked mode (n_stack > 1, not GROUPED): the input rows are n_stack equal
// groups of n_rows rows, each quantized on its own and written as output rows
// [s * n_cols, (s + 1) * n_cols).
// Threads per column-wise workgroup.  Wide RTNE tiles are shared by 8 waves
// (each quantizes 2 of the 16 row-blocks): their LDS transpose tile (52 KiB)
// then holds 8 waves instead of 4, so the VGPR budget (<= 128, 4 waves per
// SIMD) rather than LDS bounds occupancy.  The stochastic-rounding kernels
// need more registers (3 waves per SIMD) and keep 4 waves per tile, and so
// do the E2M1 grids, whose rounding is the longer instruction sequence (the
// 8-wave tile measured 1.45x slower there).
template <int GRID, int CW, int RND>
constexpr int col_threads() {
  return (GRID == kGridUniform && CW == 4 && RND == kRoundRTNE) ? 512 : 256;
}

template <int GRID, int RND, bool RHT, bool VEC, bool GROUPED, int CW>
__global__ __launch_bounds__((col_threads<GRID, CW, RND>())) void quant_cols_kernel(
    const uint16_t *__restrict__ x, int64_t n_rows, int64_t n_cols, int64_t ld,
    const int64_t *__restrict__ goff, int n_groups, int64_t n_stack, int64_t kpad,
    uint8_t *__restrict__ codes, float *__restrict__ scales, uint32_t sign_mask,
    uint32_t seed_lo, uint32_t seed_hi, uint32_t stream_id) {
  constexpr int kCols = 64 * CW;                 // tile columns
  constexpr int kTB = kColTileRows / 16;         // tile row-blocks
  constexpr int kNT = col_threads<GRID, CW, RND>();  // threads: 4 or 8 waves share the tile
  constexpr int kWaves = kNT / 64;
  constexpr int kPerWave = kTB / kWaves;         // row-blocks per wave
  static_assert(kPerWave * kWaves == kTB, "row-blocks per wave");
  // Narrow tiles prefetch the next row-block and walk down column strips;
  // wide ones hold twice the columns per lane, so they load one row-block at
  // a time (occupancy hides the latency) and interleave 4 row bands.
  constexpr bool kPrefetch = CW == 2;
  constexpr int kOrd = CW == 2 ? 1 : 4;
  constexpr int kTabs = GROUPED ? kMaxGroups + 1 : 1;
  __shared__ int64_t s_off[kTabs];
  __shared__ int64_t s_poff[kTabs];
  __shared__ int64_t s_scan[GROUPED ? kNT : 1];
  __shared__ uint2 s_codes[kCols][kTB + 1];
  __shared__ float s_scales[kCols][kTB + 1];

  int64_t padded_end;
  if (GROUPED) {
    load_group_tables<kNT>(goff, n_groups, n_rows, s_off, s_poff, s_scan);
    padded_end = s_poff[n_groups];
  } else {
    padded_end = (n_rows + 15) / 16 * 16;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t kblocks = kpad / 16;
  const int64_t n_ptiles = (kpad + kColTileRows - 1) / kColTileRows;
  const int64_t n_ctiles = (n_cols + kCols - 1) / kCols;
  const int64_t per_stack = n_ptiles * n_ctiles;
  const int64_t total = per_stack * n_stack;

  // Row range of padded block p: [row0, row0 + valid), wave-uniform.
  auto block_rows = [&](int64_t p, int64_t &row0, int &valid) {
    row0 = 0;
    valid = 0;
    if (p < kblocks && 16 * p < padded_end) {
      if (GROUPED) {
        const int e = find_group(s_poff, n_groups, 16 * p);
        row0 = s_off[e] + (16 * p - s_poff[e]);
        const int64_t left = s_off[e + 1] - row0;
        valid = left >= 16 ? 16 : (int)(left > 0 ? left : 0);
      } else {
        row0 = 16 * p;
        const int64_t left = n_rows - row0;
        valid = left >= 16 ? 16 : (int)left;
      }
    }
    row0 = uniform64(row0);
    valid = __builtin_amdgcn_readfirstlane(valid);
  };

  for (int64_t tile_all = xcd_major_block(); tile_all < total; tile_all += gridDim.x) {
    const int64_t si = tile_all / per_stack;
    int64_t pt, ct;
    col_tile_coords(tile_all - si * per_stack, n_ptiles, n_ctiles, kOrd, pt, ct);
    const uint16_t *xs = x + si * n_rows * ld;
    const int64_t out_row0 = si * n_cols;          // first output row of this stack
    const int64_t pb0 = pt * kTB;                   // first padded block of the tile
    const int64_t col0 = ct * kCols;
    const int64_t col = col0 + CW * lane;
    uint32_t keep[CW / 2];
#pragma unroll
    for (int c = 0; c < CW / 2; ++c) {
      const int64_t cc = col + 2 * c;
      keep[c] = (cc + 1 < n_cols) ? 0xFFFFFFFFu : (cc < n_cols ? 0x0000FFFFu : 0u);
    }
    const int colb = (int)(col * 2);
    // Wave w quantizes row-blocks w, w + kWaves, ... of the tile.
    uint32_t cur[16][CW / 2], nxt[16][CW / 2];
    int64_t row0;
    int valid;
    block_rows(pb0 + wave, row0, valid);
    load_col_rows<VEC, CW>(xs, ld, n_cols, row0, valid, colb, keep, cur);
#pragma unroll 1
    for (int q = 0; q < kPerWave; ++q) {
      const int rb = wave + kWaves * q;               // block within the tile (wave-uniform)
      const int64_t p = pb0 + rb;                     // padded block index
      if (kPrefetch && q < kPerWave - 1) {
        block_rows(p + kWaves, row0, valid);
        load_col_rows<VEC, CW>(xs, ld, n_cols, row0, valid, colb, keep, nxt);
      }
#pragma unroll
      for (int c = 0; c < CW / 2; ++c) {
        float va[16], vb[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          va[j] = bf16_lo(cur[j][c], RHT ? sign_bit(sign_mask, j) : 0u);
          vb[j] = bf16_hi(cur[j][c], RHT ? sign_bit(sign_mask, j) : 0u);
        }
        uint32_t a0, a1, b0, b1;
        float sa, sb;
        const uint64_t base_a =
            (uint64_t)(out_row0 + col + 2 * c) * (uint64_t)kpad + (uint64_t)p * 16u;
        const uint64_t base_b = base_a + (uint64_t)kpad;
        quantize_block<GRID, RND, RHT>(va, base_a, seed_lo, seed_hi, stream_id, a0, a1, sa);
        quantize_block<GRID, RND, RHT>(vb, base_b, seed_lo, seed_hi, stream_id, b0, b1, sb);
        s_codes[CW * lane + 2 * c][rb] = make_uint2(a0, a1);
        s_codes[CW * lane + 2 * c + 1][rb] = make_uint2(b0, b1);
        s_scales[CW * lane + 2 * c][rb] = sa;
        s_scales[CW * lane + 2 * c + 1][rb] = sb;
      }
      if (q < kPerWave - 1) {
        if (kPrefetch) {
#pragma unroll
          for (int j = 0; j < 16; ++j)
#pragma unroll
            for (int c = 0; c < CW / 2; ++c) cur[j][c] = nxt[j][c];
        } else {
          block_rows(p + kWaves, row0, valid);
          load_col_rows<VEC, CW>(xs, ld, n_cols, row0, valid, colb, keep, cur);
        }
      }
    }
    __syncthreads();
    // write back: kCols columns x 16 blocks of 8-byte codes; 16 consecutive
    // lanes write one column's 128 contiguous bytes
    constexpr int kColStep = kNT / 16;                 // columns per pass
    const int nb = (int)((kblocks - pb0) < kTB ? (kblocks - pb0) : kTB);
    const int blk = tid & 15;
    const int c0 = tid >> 4;                           // 0..kColStep-1, then +kColStep
    uint8_t *dq = codes + (out_row0 + col0 + c0) * (kpad / 2) + (pb0 + blk) * 8;
    float *ds = scales + (out_row0 + col0 + c0) * kblocks + pb0 + blk;
    const int64_t step_q = kColStep * (kpad / 2), step_s = kColStep * kblocks;
#pragma unroll
    for (int it = 0; it < kCols / kColStep; ++it) {
      const int c = c0 + kColStep * it;
      if (col0 + c < n_cols && blk < nb) {
        // streaming stores: a later kernel reads the operand
        const uint2 cv = s_codes[c][blk];
        __builtin_nontemporal_store(((uint64_t)cv.y << 32) | cv.x, reinterpret_cast<uint64_t *>(dq));
        __builtin_nontemporal_store(s_scales[c][blk], ds);
      }
      dq += step_q;
      ds += step_s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Dual-axis: one read of x gives both operands of a tensor -- the row-wise
// one (blocks along the contiguous dimension, as the row-wise kernels write
// it) and the transposed column-wise one (as quant_cols_kernel, with the same
// tiles, groups and stacking).  Each lane's two columns x 16 rows of the
// current row-block also go to a per-wave LDS buffer; read back as 16 rows x
// 8 blocks of 16 columns, they give the row-wise blocks: lane l takes row l/4
// and blocks 2(l%4), 2(l%4)+1 of the tile's 128 columns.  Each output is
// bit-identical to the single-axis call with the same options; the bf16 input
// is read once instead of twice.
// ---------------------------------------------------------------------------
template <int GRID, int RND>
__device__ __forceinline__ void quantize_block_rt(bool rht, float (&v)[16], uint64_t idx0,
                                                  uint32_t seed_lo, uint32_t seed_hi,
                                                  uint32_t stream_id, uint32_t &w0, uint32_t &w1,
                                                  float &s) {
  if (rht)
    quantize_block<GRID, RND, true>(v, idx0, seed_lo, seed_hi, stream_id, w0, w1, s);
  else
    quantize_block<GRID, RND, false>(v, idx0, seed_lo, seed_hi, stream_id, w0, w1, s);
}

// 8 dwords (16 bf16 along the block) -> FP32 with the RHT signs of `mask`
// (0 when the side has no RHT).
__device__ __forceinline__ void unpack_block(const uint4 a0, const uint4 a1, uint32_t mask,
                                             float (&v)[16]) {
  const uint32_t w[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = bf16_lo(w[i], sign_bit(mask, 2 * i));
    v[2 * i + 1] = bf16_hi(w[i], sign_bit(mask, 2 * i + 1));
  }
}

template <int GRID, int RND, bool VEC, bool GROUPED>
__global__ __launch_bounds__(256) void quant_dual_kernel(const DualArgs a, int64_t n_rows,
                                                         int64_t n_stack) {
  constexpr int kTrStride = 68;                     // dwords per staged row (64 + 4 pad)
  // Grouped: the group tables, n_groups + 1 entries each, in dynamic LDS
  // sized by the launch, so that a few groups leave room for three
  // workgroups per CU (the occupancy registers allow) where tables for the
  // 1024-group maximum would leave two.
  extern __shared__ int64_t s_tabs[];
  int64_t *const s_off = s_tabs;
  int64_t *const s_poff = s_tabs + (a.n_groups + 1);
  __shared__ int64_t s_scan[GROUPED ? 256 : 1];
  __shared__ uint2 s_codes[kColTileCols][kColTileRows / 16 + 1];
  __shared__ float s_scales[kColTileCols][kColTileRows / 16 + 1];
  __shared__ __attribute__((aligned(16))) uint32_t s_tr[4][16 * kTrStride];

  const int64_t n_cols = a.n_cols, ld = a.ld, kpad = a.kpad_c;
  int64_t padded_end;
  if (GROUPED) {
    load_group_tables(a.goff, a.n_groups, n_rows, s_off, s_poff, s_scan);
    padded_end = s_poff[a.n_groups];
  } else {
    padded_end = (n_rows + 15) / 16 * 16;
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t kblocks = kpad / 16;
  const int64_t kblocks_r = a.kpad_r / 16;
  const bool pair_aligned = (a.kpad_r % 32) == 0;   // 16-byte code / 8-byte scale pairs
  const int64_t n_ptiles = (kpad + kColTileRows - 1) / kColTileRows;
  const int64_t n_ctiles = (n_cols + kColTileCols - 1) / kColTileCols;
  const int64_t per_stack = n_ptiles * n_ctiles;
  const int64_t total = per_stack * n_stack;
  uint32_t *tr = s_tr[wave];
  const int rr = lane >> 2, c2 = lane & 3;            // row-wise: row and block pair

  auto block_rows = [&](int64_t p, int64_t &row0, int &valid) {
    row0 = 0;
    valid = 0;
    if (p < kblocks && 16 * p < padded_end) {
      if (GROUPED) {
        const int e = find_group(s_poff, a.n_groups, 16 * p);
        row0 = s_off[e] + (16 * p - s_poff[e]);
        const int64_t left = s_off[e + 1] - row0;
        valid = left >= 16 ? 16 : (int)(left > 0 ? left : 0);
      } else {
        row0 = 16 * p;
        const int64_t left = n_rows - row0;
        valid = left >= 16 ? 16 : (int)left;
      }
    }
    row0 = uniform64(row0);
    valid = __builtin_amdgcn_readfirstlane(valid);
  };

  // Each XCD takes a contiguous range of the row-band-major tile order (the
  // launcher makes the grid a multiple of 8), so the tiles it runs together
  // share input rows and output lines in its L2 (MoE-124B X: 3.18 -> 3.05 ms).
  for (int64_t tile_all = xcd_major_block(); tile_all < total; tile_all += gridDim.x) {
    const int64_t si = tile_all / per_stack;
    const int64_t tile = tile_all - si * per_stack;
    const int64_t pt = tile / n_ctiles;
    const int64_t ct = tile - pt * n_ctiles;
    const uint16_t *xs = a.x + si * n_rows * ld;
    const int64_t out_row0 = si * n_cols;
    const int64_t pb0 = pt * (kColTileRows / 16);
    const int64_t col0 = ct * kColTileCols;
    const int64_t col = col0 + 2 * lane;
    const uint32_t keep = (col + 1 < n_cols) ? 0xFFFFFFFFu : (col < n_cols ? 0x0000FFFFu : 0u);
    const int col2 = (int)(col * 2);
    const int64_t kbr0 = col0 / 16 + 2 * c2;           // this lane's first row-wise block
    uint32_t cur[16], nxt[16];
    int64_t row0, nrow0;
    int valid, nvalid;
    block_rows(pb0 + wave, row0, valid);
    load_col_block<VEC>(xs, ld, n_cols, row0, valid, col2, keep, cur);
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
      const int rb = wave + 4 * q;
      const int64_t p = pb0 + rb;
      if (q < 3) {
        block_rows(p + 4, nrow0, nvalid);
        load_col_block<VEC>(xs, ld, n_cols, nrow0, nvalid, col2, keep, nxt);
      }
      // stage the raw dwords for the row-wise side
#pragma unroll
      for (int j = 0; j < 16; ++j) tr[j * kTrStride + lane] = cur[j];
      __builtin_amdgcn_wave_barrier();
      const uint4 *trr = reinterpret_cast<const uint4 *>(tr + rr * kTrStride + 16 * c2);
      const uint4 r0 = trr[0], r1 = trr[1], r2 = trr[2], r3 = trr[3];
      __builtin_amdgcn_wave_barrier();

      // column-wise side (transposed output through LDS, as quant_cols_kernel)
      {
        float va[16], vb[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          va[j] = bf16_lo(cur[j], sign_bit(a.mask_c, j));
          vb[j] = bf16_hi(cur[j], sign_bit(a.mask_c, j));
        }
        uint32_t a0, a1, b0, b1;
        float sa, sb;
        const uint64_t base_a = (uint64_t)(out_row0 + col) * (uint64_t)kpad + (uint64_t)p * 16u;
        const uint64_t base_b = base_a + (uint64_t)kpad;
        quantize_block_rt<GRID, RND>(a.rht_c, va, base_a, a.seed_lo, a.seed_hi, a.sid_c, a0, a1,
                                     sa);
        quantize_block_rt<GRID, RND>(a.rht_c, vb, base_b, a.seed_lo, a.seed_hi, a.sid_c, b0, b1,
                                     sb);
        s_codes[2 * lane][rb] = make_uint2(a0, a1);
        s_codes[2 * lane + 1][rb] = make_uint2(b0, b1);
        s_scales[2 * lane][rb] = sa;
        s_scales[2 * lane + 1][rb] = sb;
      }

      // row-wise side: row row0 + rr, blocks kbr0 and kbr0 + 1
      if (rr < valid && kbr0 < kblocks_r) {
        const int64_t grow = si * n_rows + row0 + rr;
        const bool two = kbr0 + 1 < kblocks_r;
        float v[16];
        uint32_t w0, w1, w2 = 0, w3 = 0;
        float s0, s1 = 0.0f;
        unpack_block(r0, r1, a.mask_r, v);
        quantize_block_rt<GRID, RND>(a.rht_r, v, (uint64_t)(grow * a.kpad_r + kbr0 * 16),
                                     a.seed_lo, a.seed_hi, a.sid_r, w0, w1, s0);
        if (two) {
          unpack_block(r2, r3, a.mask_r, v);
          quantize_block_rt<GRID, RND>(a.rht_r, v, (uint64_t)(grow * a.kpad_r + kbr0 * 16 + 16),
                                       a.seed_lo, a.seed_hi, a.sid_r, w2, w3, s1);
        }
        uint8_t *cq = a.codes_r + grow * (a.kpad_r / 2) + kbr0 * 8;
        float *cs = a.scales_r + grow * kblocks_r + kbr0;
        if (two && pair_aligned) {
          *reinterpret_cast<uint4 *>(cq) = make_uint4(w0, w1, w2, w3);
          *reinterpret_cast<float2 *>(cs) = make_float2(s0, s1);
        } else {
          *reinterpret_cast<uint2 *>(cq) = make_uint2(w0, w1);
          cs[0] = s0;
          if (two) {
            *reinterpret_cast<uint2 *>(cq + 8) = make_uint2(w2, w3);
            cs[1] = s1;
          }
        }
      }
      if (q < 3) {
        row0 = nrow0;
        valid = nvalid;
#pragma unroll
        for (int j = 0; j < 16; ++j) cur[j] = nxt[j];
      }
    }
    __syncthreads();
    const int nb = (int)((kblocks - pb0) < 16 ? (kblocks - pb0) : 16);
    const int blk = tid & 15;
    const int c0 = tid >> 4;
    uint8_t *dq = a.codes_c + (out_row0 + col0 + c0) * (kpad / 2) + (pb0 + blk) * 8;
    float *ds = a.scales_c + (out_row0 + col0 + c0) * kblocks + pb0 + blk;
    const int64_t step_q = 16 * (kpad / 2), step_s = 16 * kblocks;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int c = c0 + 16 * it;
      if (col0 + c < n_cols && blk < nb) {
        // streaming stores, as the column-wise kernel's: 128-byte code pieces
        // that no later access in this kernel touches (2^28 elements, RTNE:
        // 277 -> 204 us; the row-wise side's 64-byte pieces, whose other half
        // a neighbouring tile writes, stay ordinary stores, which measured
        // faster for them)
        const uint2 cv = s_codes[c][blk];
        __builtin_nontemporal_store(((uint64_t)cv.y << 32) | cv.x, reinterpret_cast<uint64_t *>(dq));
        __builtin_nontemporal_store(s_scales[c][blk], ds);
      }
      dq += step_q;
      ds += step_s;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Dequantizer: one lane per block.  value = (float)((double)(sign*L) *
// (double)s / g); with the inverse RHT the FP64 block goes back through
// (1/4) D H16 (same butterfly order) before the cast.
// ---------------------------------------------------------------------------
template <int GRID, bool INV>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ codes,
                                                      const float *__restrict__ scales,
                                                      int64_t rows, int64_t kblocks,
                                                      float *__restrict__ out, int64_t ld_out,
                                                      uint32_t sign_mask) {
  const int64_t nblk = rows * kblocks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < nblk; b += stride) {
    const int64_t row = b / kblocks;
    const int64_t kb = b - row * kblocks;
    const uint2 c = *reinterpret_cast<const uint2 *>(codes + b * 8);
    const double s = (double)scales[b];
    constexpr double g = (double)grid_g<GRID>();
    double d[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t w = j < 8 ? c.x : c.y;
      const uint32_t n = (w >> (4 * (j & 7))) & 0xFu;
      const uint32_t mi = n & 7u;
      double lv;
      if (GRID == kGridUniform) {
        lv = (double)mi;
      } else {
        lv = mi < 4 ? 0.5 * (double)mi : (mi == 4 ? 2.0 : (mi == 5 ? 3.0 : (mi == 6 ? 4.0 : 6.0)));
      }
      if (n & 8u) lv = -lv;
      d[j] = lv * s / g;
    }
    if (INV) {
#pragma unroll
      for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if ((i & h) == 0) {
            const double a = d[i], bb = d[i + h];
            d[i] = a + bb;
            d[i + h] = a - bb;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        d[j] *= 0.25;
        if ((sign_mask >> j) & 1u) d[j] = -d[j];
      }
    }
    float *o = out + row * ld_out + kb * 16;
#pragma unroll
    for (int j = 0; j < 16; ++j) o[j] = (float)d[j];
  }
}

// ---------------------------------------------------------------------------
// Launchers (host side).  Grids are sized to a few waves of workgroups per CU
// and the kernels grid-stride, so any size runs with bounded launches.
// ---------------------------------------------------------------------------
static int grid_for(int64_t work_items, int per_block, int max_blocks) {
  int64_t b = (work_items + per_block - 1) / per_block;
  if (b > max_blocks) b = max_blocks;
  if (b < 1) b = 1;
  return (int)b;
}

// Compute units of the current device, queried once per device.
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int GRID, int RND, bool RHT>
static hipError_t launch_rows_t(const QuantArgs &a, hipStream_t st) {
  const int64_t kblocks = a.kpad / 16;
  const bool aligned = (reinterpret_cast<uintptr_t>(a.x) & 15u) == 0;
  if (aligned && a.ld == a.n_cols && a.n_cols % 16 == 0) {
    const int64_t nblk = a.n_rows * kblocks;
    // A persistent-style grid: with round-to-nearest the loop is bound by
    // HBM and two workgroups per CU keep enough loads in flight; the Philox
    // draws of stochastic rounding make it ALU-heavier, so it gets four.
    const int per_cu = RND == kRoundSR ? 4 : 2;
    const int blocks = grid_for(nblk, 256, per_cu * device_cus());
    hipLaunchKernelGGL((quant_rows_contig_kernel<GRID, RND, RHT>), dim3(blocks), dim3(256), 0, st,
                       a.x, nblk, a.codes, a.scales, a.sign_mask, a.seed_lo, a.seed_hi,
                       a.stream_id);
    return hipGetLastError();
  }
  const int gx = grid_for(kblocks, 256, 64);
  const int gy = (int)(a.n_rows < 8192 ? a.n_rows : 8192);
  if (aligned && a.ld % 8 == 0)
    hipLaunchKernelGGL((quant_rows_kernel<GRID, RND, RHT, true>), dim3(gx, gy), dim3(256), 0, st,
                       a.x, a.n_rows, a.n_cols, a.ld, kblocks, a.codes, a.scales, a.sign_mask,
                       a.seed_lo, a.seed_hi, a.stream_id);
  else
    hipLaunchKernelGGL((quant_rows_kernel<GRID, RND, RHT, false>), dim3(gx, gy), dim3(256), 0, st,
                       a.x, a.n_rows, a.n_cols, a.ld, kblocks, a.codes, a.scales, a.sign_mask,
                       a.seed_lo, a.seed_hi, a.stream_id);
  return hipGetLastError();
}

template <int GRID, int RND, bool RHT, int CW>
static hipError_t launch_cols_cw(const QuantArgs &a, bool vec, hipStream_t st) {
  const int64_t n_ptiles = (a.kpad + kColTileRows - 1) / kColTileRows;
  const int64_t n_ctiles = (a.n_cols + 64 * CW - 1) / (64 * CW);
  const int64_t n_stack = a.axis == 2 ? a.n_groups : 1;
  const int64_t rows_per = a.n_rows / n_stack;
  int blocks = grid_for(n_ptiles * n_ctiles * n_stack, 1, 256 * 16);
  if (blocks >= 8) blocks -= blocks % 8;   // whole XCD rounds (xcd_major_block)
#define UFP4_QC(V, G)                                                                          \
  hipLaunchKernelGGL((quant_cols_kernel<GRID, RND, RHT, V, G, CW>), dim3(blocks),                \
                     dim3(col_threads<GRID, CW, RND>()), 0,                                      \
                     st, a.x, rows_per, a.n_cols, a.ld, a.goff, a.n_groups, n_stack, a.kpad,    \
                     a.codes, a.scales, a.sign_mask, a.seed_lo, a.seed_hi, a.stream_id)
  const bool grouped = a.goff != nullptr;
  if (vec) {
    if (grouped) UFP4_QC(true, true); else UFP4_QC(true, false);
  } else {
    if (grouped) UFP4_QC(false, true); else UFP4_QC(false, false);
  }
#undef UFP4_QC
  return hipGetLastError();
}

template <int GRID, int RND, bool RHT>
static hipError_t launch_cols_t(const QuantArgs &a, hipStream_t st) {
  const uintptr_t xa = reinterpret_cast<uintptr_t>(a.x);
  // Four columns per lane need 8-byte loads: 8-byte aligned rows and a column
  // count that is a multiple of 4 (so no load straddles the end of a row).
  // They pay off once there are enough wide tiles to fill the GPU several
  // times over; smaller inputs keep two columns per lane.
  const bool vec4 = (xa & 7u) == 0 && a.ld % 4 == 0 && a.n_cols % 4 == 0;
  const int64_t n_stack = a.axis == 2 ? a.n_groups : 1;
  const int64_t wide_tiles =
      ((a.kpad + kColTileRows - 1) / kColTileRows) * ((a.n_cols + 255) / 256) * n_stack;
  if (vec4 && wide_tiles >= 8 * (int64_t)device_cus())
    return launch_cols_cw<GRID, RND, RHT, 4>(a, true, st);
  // dword loads need 4-byte aligned rows and an even column count (a dword
  // straddling the last column of the last row would read as zero)
  const bool vec = (xa & 3u) == 0 && a.ld % 2 == 0 && a.n_cols % 2 == 0;
  return launch_cols_cw<GRID, RND, RHT, 2>(a, vec, st);
}

template <int GRID, int RND>
static hipError_t launch_q2(const QuantArgs &a, hipStream_t st) {
  if (a.axis == 0)
    return a.rht ? launch_rows_t<GRID, RND, true>(a, st) : launch_rows_t<GRID, RND, false>(a, st);
  return a.rht ? launch_cols_t<GRID, RND, true>(a, st) : launch_cols_t<GRID, RND, false>(a, st);
}

hipError_t launch_quantize(const QuantArgs &a, hipStream_t st) {
  if (a.grid == kGridUniform)
    return a.rnd == kRoundSR ? launch_q2<kGridUniform, kRoundSR>(a, st)
                             : launch_q2<kGridUniform, kRoundRTNE>(a, st);
  if (a.grid == kGridE2M1)
    return a.rnd == kRoundSR ? launch_q2<kGridE2M1, kRoundSR>(a, st)
                             : launch_q2<kGridE2M1, kRoundRTNE>(a, st);
  return a.rnd == kRoundSR ? launch_q2<kGridE2M1Max2, kRoundSR>(a, st)
                           : launch_q2<kGridE2M1Max2, kRoundRTNE>(a, st);
}

template <int GRID, int RND>
static hipError_t launch_dual_t(const DualArgs &a, hipStream_t st) {
  const int64_t n_ptiles = (a.kpad_c + kColTileRows - 1) / kColTileRows;
  const int64_t n_ctiles = (a.n_cols + kColTileCols - 1) / kColTileCols;
  const int64_t n_stack = a.col_axis == 2 ? a.n_groups : 1;
  const int64_t rows_per = a.n_rows / n_stack;
  // A grid of up to 16384 workgroups (64 per CU over the launch, a few at a
  // time), each taking every gridDim-th tile: more, shorter-lived
  // workgroups keep the tiles in flight closer together.
  // Measured over the bench shapes against caps of 768 to 65536: 16384 was
  // best or within 2 % everywhere (MoE-124B X 3.08 -> 2.80 ms, W 0.32 ->
  // 0.30 ms, MoE-7.9B dY 0.27 -> 0.23 ms, 2^28 0.20 -> 0.19 ms); larger
  // grids repeat the group-table set-up per workgroup too often.
  int blocks = grid_for(n_ptiles * n_ctiles * n_stack, 1, 256 * 64);
  if (blocks >= 8) blocks -= blocks % 8;   // whole XCD rounds (xcd_major_block)
  const bool vec = ((reinterpret_cast<uintptr_t>(a.x) & 3u) == 0) && (a.ld % 2 == 0) &&
                   (a.n_cols % 2 == 0);
  const bool grouped = a.goff != nullptr;
  // the group tables' dynamic LDS (at most 16.4 KB: with the static 45.5 KB
  // the workgroup stays within 64 KB)
  const size_t tabs = grouped ? 2 * (size_t)(a.n_groups + 1) * sizeof(int64_t) : 0;
#define UFP4_QD(V, G) \
  hipLaunchKernelGGL((quant_dual_kernel<GRID, RND, V, G>), dim3(blocks), dim3(256), tabs, st, a, \
                     rows_per, n_stack)
  if (vec) {
    if (grouped) UFP4_QD(true, true); else UFP4_QD(true, false);
  } else {
    if (grouped) UFP4_QD(false, true); else UFP4_QD(false, false);
  }
#undef UFP4_QD
  return hipGetLastError();
}

hipError_t launch_quantize_dual(const DualArgs &a, hipStream_t st) {
  if (a.grid == kGridUniform)
    return a.rnd == kRoundSR ? launch_dual_t<kGridUniform, kRoundSR>(a, st)
                             : launch_dual_t<kGridUniform, kRoundRTNE>(a, st);
  if (a.grid == kGridE2M1)
    return a.rnd == kRoundSR ? launch_dual_t<kGridE2M1, kRoundSR>(a, st)
                             : launch_dual_t<kGridE2M1, kRoundRTNE>(a, st);
  return a.rnd == kRoundSR ? launch_dual_t<kGridE2M1Max2, kRoundSR>(a, st)
                           : launch_dual_t<kGridE2M1Max2, kRoundRTNE>(a, st);
}

hipError_t launch_dequantize(const uint8_t *codes, const float *scales, int64_t rows,
                             int64_t kpad, int grid, bool inverse, uint32_t sign_mask, float *out,
                             int64_t ld_out, hipStream_t st) {
  const int64_t kblocks = kpad / 16;
  const int blocks = grid_for(rows * kblocks, 256, 256 * 16);
#define UFP4_DQ(G, I)                                                                      \
  hipLaunchKernelGGL((dequant_kernel<G, I>), dim3(blocks), dim3(256), 0, st, codes, scales, \
                     rows, kblocks, out, ld_out, sign_mask)
  if (grid == kGridUniform) {
    if (inverse) UFP4_DQ(kGridUniform, true); else UFP4_DQ(kGridUniform, false);
  } else if (grid == kGridE2M1) {
    if (inverse) UFP4_DQ(kGridE2M1, true); else UFP4_DQ(kGridE2M1, false);
  } else {
    if (inverse) UFP4_DQ(kGridE2M1Max2, true); else UFP4_DQ(kGridE2M1Max2, false);
  }
#undef UFP4_DQ
  return hipGetLastError();
}

}  // namespace ufp4
