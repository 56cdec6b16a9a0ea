// Block-scaled 4-bit GEMM, C = A_hat * B_hat^T, on CDNA4 MFMA (gfx950).
//
// Method: the low-precision training GEMMs consume the rotated quantized
// operands and contract along the dimension they were quantized and rotated
// along ("Rethinking Shrinkage Bias in LLM FP4 Pretraining", arXiv
// 2606.20381, paperlayer.ai summary, section 2 "Random Hadamard transforms").
// With codes q and FP32 block scales s per 16 elements:
//   C[m,n] = (1/g^2) * sum_kb sa[m,kb] * sb[n,kb] * P_kb[m,n],
//   P_kb[m,n] = sum_{k in kb} qa[m,k] * qb[n,k]   (an exact small integer).
//
// Design for gfx950: every grid level is an exact FP8 E4M3 value (uniform:
// 0..7; E2M1 doubled: 0,1,2,3,4,6,8,12), so one v_mfma_f32_32x32x16_fp8_fp8
// per 16-element block yields P_kb exactly in FP32 (|P| <= 16*144).  The
// scale products sa[m,kb]*sb[n,kb] of a wave's 32 x 64 outputs are one FP32
// outer product, computed by v_mfma_f32_32x32x1_2b_f32 (K = 1, the A column
// broadcast to both 32-column blocks): an exact product rounded once, the
// same value as an FP32 multiply, in the same lane/register layout as P.
// What remains on the vector ALU is one FMA per output per block,
// acc += S * P.  Per 32x32 tile and block the matrix core thus spends 32 + 32
// cycles; on gfx950 the vector work of the other waves on a SIMD overlaps
// that only a little, so the two add up, and staging, LDS fragment reads,
// the barrier and waits on MFMA results come on top.  Nibbles are expanded
// to FP8 (v_perm_b32 look-up) once per workgroup while staging into LDS, so
// the waves read ready MFMA operands.
//
// Tiling: 512 threads = 8 waves, 128 x 128 output tile; the waves form a
// 4 x 2 grid and wave (wm, wn) owns rows [32wm, 32wm+32) x columns
// [64wn, 64wn+64) = two 32x32 MFMA tiles sharing one A fragment and one
// scale outer product per block.  The kernel is built for 4 waves per SIMD
// (at most 128 VGPRs, two workgroups per CU) so that a SIMD has other waves
// to issue while one waits on MFMA results, LDS or the barrier.  K advances
// 64 (4 blocks) per LDS stage, double-buffered: the global loads of stage
// s+1 are in flight while stage s is computed, and there is one barrier per
// stage; the stage loop is unrolled by two so each half addresses its LDS
// buffer with constant offsets.  Operands are read with buffer loads whose
// range check returns zero past the tile's rows, so ragged edges need no
// branches; full stages carry the stage offset in the scalar offset, and
// only the last, partial stage tests each lane's block against the K range.
// The four blocks of a stage are unrolled (LDS offsets become immediates);
// an empty asm ties each block's fragments to the previous block's
// accumulators, so the compiler issues a block's MFMAs only after the
// previous block's FMAs instead of hoisting every block's MFMAs and holding
// all their products in registers.
// Tiles are assigned XCD-major: the 8 XCDs each walk a contiguous range of
// tiles, so a row panel of A stays in one L2.  Outputs are written with
// nontemporal (streaming) stores.  A contraction longer than 65536 elements
// is accumulated in chunks of that length: at the end of each chunk the
// tile's FP32 sums are added to its outputs (read back by the same lanes),
// so the error of the FP32 running sum stays that of a 65536-long chain
// whatever K is; shorter contractions write once and are unchanged.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "ufp4_device.h"
#include "ufp4_kernels.h"

namespace ufp4 {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx32 __attribute__((ext_vector_type(32)));

constexpr int kThreads = 512;
constexpr int kWavesM = 4;                    // waves along M
constexpr int kNT = 2;                        // 32-column MFMA tiles per wave
constexpr int kBM = 32 * kWavesM;             // 128
constexpr int kBN = 32 * kNT * (kThreads / 64 / kWavesM);   // 128
constexpr int kSB = 4;                        // 16-element blocks per stage
constexpr int kSBLog = 2;
constexpr int kRowBytes = kSB * 16 + 8;       // FP8 bytes per LDS row (+8 breaks bank aliasing)
constexpr int kAItems = kBM * kSB / kThreads; // (row, block) items per thread: 1
constexpr int kBItems = kBN * kSB / kThreads; // 1
static_assert(kAItems * kThreads == kBM * kSB && kBItems * kThreads == kBN * kSB, "staging");
static_assert((1 << kSBLog) == kSB, "kSBLog");
static_assert(kAItems == 1 && kBItems == 1, "one A and one B staging item per thread");
constexpr int kMaxGemmGroups = 1024;
constexpr int kXcds = 8;
// A tile's FP32 running sums go to its outputs every kFlushStages stages
// (65536 K-elements): one FP32 chain over 2^20 blocks of same-signed
// products drifts by about 1e-3 of the result, chunks of 4096 blocks by
// about 1e-7.
constexpr int kFlushStages = 1024;
static_assert((kFlushStages & (kFlushStages - 1)) == 0 && kFlushStages % 2 == 0, "flush");

struct Stage {
  uint8_t a[kBM * kRowBytes];
  uint8_t b[kBN * kRowBytes];
  // block-major scales sa[blk][row]; the 16-entry pad per block puts the four
  // blocks of a row, which a quarter-wave stores together, in different banks
  float sa[kSB * (kBM + 16)];
  float sb[kSB * (kBN + 16)];
};

// 8 nibbles -> 8 FP8 E4M3 bytes.  Output byte order [n0 n2 n4 n6 | n1 n3 n5
// n7]; A and B use the same order, so products still pair up.
template <int GRID>
__device__ __forceinline__ uint2 nib8_to_fp8(uint32_t w) {
  constexpr uint32_t lut_lo = 0x44403800u;  // 0, 1, 2, 3
  constexpr uint32_t lut_hi = (GRID == kGridUniform) ? 0x4E4C4A48u   // 4, 5, 6, 7
                                                     : 0x54504C48u;  // 4, 6, 8, 12
  const uint32_t me = w & 0x07070707u;
  const uint32_t mo = (w >> 4) & 0x07070707u;
  const uint32_t fe = __builtin_amdgcn_perm(lut_hi, lut_lo, me) | ((w << 4) & 0x80808080u);
  const uint32_t fo = __builtin_amdgcn_perm(lut_hi, lut_lo, mo) | (w & 0x80808080u);
  return make_uint2(fe, fo);
}

struct TileJob {
  int64_t a_row0, a_rows;   // A rows [a_row0, a_row0 + a_rows)
  int64_t b_row0, b_rows;
  int64_t kb0, kb1;         // block range [kb0, kb1)
  int64_t c_off;            // element offset of C(0, 0) of the tile
};

// Per-thread staging registers of one stage.
struct Regs {
  uint2 aq[kAItems];
  float as[kAItems];
  uint2 bq[kBItems];
  float bs[kBItems];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int n = bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0 : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

template <int GRID>
struct Gemm {
  const GemmArgs &g;
  TileJob job;
  __amdgpu_buffer_rsrc_t ra_q, ra_s, rb_q, rb_s;
  int nkb;     // blocks in [kb0, kb1)
  int oq, os;  // this thread's (row, block) item at stage 0: code and scale byte offsets

  __device__ Gemm(const GemmArgs &args, const TileJob &j) : g(args), job(j) {
    const int64_t kblocks = g.kpad / 16;
    // Resources start at the tile's first row, so 32-bit offsets suffice and
    // rows past the tile read as zero.
    ra_q = make_rsrc(g.a_codes + job.a_row0 * (g.kpad / 2), job.a_rows * (g.kpad / 2));
    ra_s = make_rsrc(g.a_scales + job.a_row0 * kblocks, job.a_rows * kblocks * 4);
    rb_q = make_rsrc(g.b_codes + job.b_row0 * (g.kpad / 2), job.b_rows * (g.kpad / 2));
    rb_s = make_rsrc(g.b_scales + job.b_row0 * kblocks, job.b_rows * kblocks * 4);
    nkb = (int)(job.kb1 - job.kb0);
    int row = threadIdx.x >> kSBLog;
    const int blk = threadIdx.x & (kSB - 1);
    // opaque per tile: the lane's row offsets are formed here for every
    // tile rather than hoisted out of the tile loop and held (spilled)
    // across the K loop
    asm volatile("" : "+v"(row));
    oq = (int)(row * (g.kpad / 2) + (job.kb0 + blk) * 8);
    os = (int)((row * kblocks + job.kb0 + blk) * 4);
  }

  // Global loads of stage st (blocks kb0 + st*kSB ...).  Full stages put the
  // stage offset in the scalar offset; only the last, partial stage needs the
  // per-lane range test (offsets past the resource read as zero).
  __device__ __forceinline__ void load(Regs &r, int st) const {
    const int kbs = st * kSB;
    int vq = oq, vs = os, sq = kbs * 8, ss = kbs * 4;
    if (kbs + kSB > nkb) {
      const bool ok = kbs + (int)(threadIdx.x & (kSB - 1)) < nkb;
      vq = ok ? oq + sq : 0x7FFFFFF8;
      vs = ok ? os + ss : 0x7FFFFFF8;
      sq = 0;
      ss = 0;
    }
    // the stage offsets are wave-uniform: keep them in scalar registers (the
    // buffer loads' scalar offset), or the compiler loops over lanes
    sq = __builtin_amdgcn_readfirstlane(sq);
    ss = __builtin_amdgcn_readfirstlane(ss);
    const auto a = __builtin_amdgcn_raw_buffer_load_b64(ra_q, vq, sq, 0);
    r.aq[0] = make_uint2(a[0], a[1]);
    r.as[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(ra_s, vs, ss, 0));
    const auto b = __builtin_amdgcn_raw_buffer_load_b64(rb_q, vq, sq, 0);
    r.bq[0] = make_uint2(b[0], b[1]);
    r.bs[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb_s, vs, ss, 0));
  }

  __device__ __forceinline__ static void store(const Regs &r, Stage &s) {
    const int row = threadIdx.x >> kSBLog, blk = threadIdx.x & (kSB - 1);
    uint2 *da = reinterpret_cast<uint2 *>(s.a + row * kRowBytes + blk * 16);
    da[0] = nib8_to_fp8<GRID>(r.aq[0].x);
    da[1] = nib8_to_fp8<GRID>(r.aq[0].y);
    s.sa[blk * (kBM + 16) + row] = r.as[0];
    uint2 *db = reinterpret_cast<uint2 *>(s.b + row * kRowBytes + blk * 16);
    db[0] = nib8_to_fp8<GRID>(r.bq[0].x);
    db[1] = nib8_to_fp8<GRID>(r.bq[0].y);
    s.sb[blk * (kBN + 16) + row] = r.bs[0];
  }

  // One stage: per block, the two 32x32 block products P (FP8 MFMA) and the
  // scale products S = sa x sb of the wave's 32 x 64 outputs (one FP32
  // outer-product MFMA), then acc += S * P with one FMA per output.
  __device__ __forceinline__ static void compute(const Stage &s, floatx16 (&acc)[kNT]) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave % kWavesM, wn = wave / kWavesM;
    const int l32 = lane & 31;
    const int half = lane >> 5;
    floatx16 zero;
#pragma unroll
    for (int r = 0; r < 16; ++r) zero[r] = 0.0f;
    floatx32 zero32;
#pragma unroll
    for (int r = 0; r < 32; ++r) zero32[r] = 0.0f;
    const uint8_t *pa = s.a + (wm * 32 + l32) * kRowBytes + 8 * half;
    const uint8_t *pb = s.b + (wn * 32 * kNT + l32) * kRowBytes + 8 * half;
    const float *psa = s.sa + wm * 32 + l32;
    const float *psb = s.sb + wn * 32 * kNT + lane;
#pragma unroll
    for (int b = 0; b < kSB; ++b) {
      long af = *reinterpret_cast<const long *>(pa + b * 16);
      long bf0 = *reinterpret_cast<const long *>(pb + b * 16);
      long bf1 = *reinterpret_cast<const long *>(pb + 32 * kRowBytes + b * 16);
      float a1 = psa[b * (kBM + 16)];
      float b1 = psb[b * (kBN + 16)];
      // this block's MFMAs may not start before the previous block's FMAs
      // are done (keeps the unrolled blocks from holding several blocks'
      // products in registers); the LDS reads above may run ahead
      asm volatile("" : "+v"(af), "+v"(bf0), "+v"(bf1), "+v"(a1), "+v"(b1)
                   : "v"(acc[0]), "v"(acc[1]));
      const floatx32 S = __builtin_amdgcn_mfma_f32_32x32x1f32(a1, b1, zero32, 1, 0, 0);
      const floatx16 p0 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(af, bf0, zero, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[0][r] = fmaf(S[r], p0[r], acc[0][r]);
      const floatx16 p1 = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(af, bf1, zero, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[1][r] = fmaf(S[16 + r], p1[r], acc[1][r]);
    }
  }

  __device__ void run(Stage *stages) {
    floatx16 acc[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[nt][r] = 0.0f;

    const int nst = (nkb + kSB - 1) / kSB;
    bool flushed = false;
    // chunks of kFlushStages stages, each a full pipeline (its first stage
    // staged before the loop); the last barrier of a chunk's loop comes
    // after every wave's last read of both LDS buffers
    for (int c0 = 0; c0 < nst; c0 += kFlushStages) {
      const int c1 = min(nst, c0 + kFlushStages);
      Regs r;
      load(r, c0);
      store(r, stages[0]);
      __syncthreads();
      // unrolled by two so that each half addresses its LDS buffer with
      // constant offsets
      for (int st = c0; st < c1; st += 2) {
        if (st + 1 < c1) load(r, st + 1);
        compute(stages[0], acc);
        if (st + 1 < c1) store(r, stages[1]);
        __syncthreads();
        if (st + 1 >= c1) break;
        if (st + 2 < c1) load(r, st + 2);
        compute(stages[1], acc);
        if (st + 2 < c1) store(r, stages[0]);
        __syncthreads();
      }
      if (c1 < nst) {
        put<true>(acc, flushed);
        flushed = true;
      }
    }
    put<false>(acc, flushed);
  }

  // Writes acc / g^2 to the tile's outputs, or adds it to what an earlier
  // flush left there.  FLUSH (a chunk of a long contraction is done): acc
  // then keeps what the output could not hold -- nothing for FP32 outputs,
  // the bf16 rounding residual for bf16 outputs (exact in FP32, scaled back
  // by g^2) -- and the next chunk accumulates on top of it.
  template <bool FLUSH>
  __device__ __forceinline__ void put(floatx16 (&acc)[kNT], bool add) {
    // 1/g^2, with the E2M1 levels doubled in FP8: 1/(2*6)^2 and 1/(2*2)^2
    constexpr float g2 = (GRID == kGridUniform) ? 49.0f : (GRID == kGridE2M1) ? 144.0f : 16.0f;
    constexpr float inv_g2 = 1.0f / g2;
    // Row offsets r -> 8*(r/4) + (r%4) are wave-uniform, so the per-lane part
    // is one pointer and one remaining-rows count.  The tile's bookkeeping
    // goes through empty asms so that the pointer and the sixteen row
    // offsets are formed here, at each flush and after the K loop, instead
    // of being hoisted and held in registers across it.
    int tid = threadIdx.x;
    int64_t ldc = g.ldc, c_off = job.c_off, a_rows = job.a_rows, b_rows = job.b_rows;
    asm volatile("" : "+v"(tid), "+s"(ldc), "+s"(c_off), "+s"(a_rows), "+s"(b_rows));
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave % kWavesM, wn = wave / kWavesM;
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const int m0 = wm * 32 + 4 * half;
    const int n0 = wn * kNT * 32 + l32;
    const int mrem = (int)a_rows - m0;
    const int nrem = (int)b_rows - n0;
    const int64_t off = c_off + m0 * ldc + n0;
    if (g.out_bf16) {
      // bf16 epilogue: the FP32 result rounded to nearest even (the bias
      // 0x7FFF + lsb carries into the kept half exactly when the dropped half
      // is above, or equal with an odd kept half; infinities stay infinite)
      uint16_t *cl = static_cast<uint16_t *>(g.c) + off;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dm = 8 * (r >> 2) + (r & 3);
          if (nt * 32 < nrem && dm < mrem) {
            uint16_t *p = cl + dm * ldc + nt * 32;
            float t = acc[nt][r] * inv_g2;
            if (add) t += __uint_as_float((uint32_t)*p << 16);
            const uint32_t u = __float_as_uint(t);
            const uint16_t h = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
            __builtin_nontemporal_store(h, p);
            if (FLUSH) acc[nt][r] = (t - __uint_as_float((uint32_t)h << 16)) * g2;
          }
        }
      }
    } else {
      float *cl = static_cast<float *>(g.c) + off;
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dm = 8 * (r >> 2) + (r & 3);
          if (nt * 32 < nrem && dm < mrem) {
            float *p = cl + dm * ldc + nt * 32;
            float t = acc[nt][r] * inv_g2;
            if (add) t += *p;
            __builtin_nontemporal_store(t, p);
          }
          if (FLUSH) acc[nt][r] = 0.0f;
        }
      }
    }
  }
};

// A wave-uniform 64-bit value held in scalar registers.
__device__ __forceinline__ int64_t wave_uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int64_t clampv(int64_t v, int64_t n) {
  return v < 0 ? 0 : (v > n ? n : v);
}

// Group tables for the grouped modes: s_off = row offsets (clamped so no
// access leaves the operands whatever the device array holds; a decreasing
// pair is an empty group), s_pre = prefix of per-group tile counts (mode 1) or
// of padded K lengths (mode 2).
template <int MODE>
__device__ void load_gemm_groups(const GemmArgs &g, int64_t *s_off, int64_t *s_pre,
                                 int64_t *s_scan, int *s_order) {
  const int tid = threadIdx.x;
  const int ng = g.n_groups;
  const int per = (ng + kThreads - 1) / kThreads;
  const int g0 = tid * per;
  const int64_t tiles_n = (g.N + kBN - 1) / kBN;
  const int64_t limit = (MODE == 1) ? g.M : (int64_t)1 << 40;
  int64_t local = 0;
  for (int e = g0; e < g0 + per && e < ng; ++e) {
    const int64_t a = clampv(g.goff[e], limit), b = clampv(g.goff[e + 1], limit);
    s_off[e] = a;
    const int64_t cnt = b > a ? b - a : 0;
    local += (MODE == 1) ? ((cnt + kBM - 1) / kBM) * tiles_n : (cnt + 15) / 16 * 16;
  }
  if (tid == 0) s_off[ng] = clampv(g.goff[ng], limit);
  s_scan[tid] = local;
  __syncthreads();
  for (int d = 1; d < kThreads; d <<= 1) {
    const int64_t add = tid >= d ? s_scan[tid - d] : 0;
    __syncthreads();
    s_scan[tid] += add;
    __syncthreads();
  }
  int64_t run = tid ? s_scan[tid - 1] : 0;
  for (int e = g0; e < g0 + per && e < ng; ++e) {
    s_pre[e] = run;
    int64_t cnt = s_off[e + 1] - s_off[e];
    cnt = cnt > 0 ? cnt : 0;
    run += (MODE == 1) ? ((cnt + kBM - 1) / kBM) * tiles_n : (cnt + 15) / 16 * 16;
  }
  if (tid == kThreads - 1) s_pre[ng] = s_scan[kThreads - 1];
  __syncthreads();
  if (MODE == 2) {
    // Largest group first: every tile of a group costs its group's K, so
    // dispatching the heaviest groups' tiles first keeps the tail short.
    // Rank by (count desc, index asc); O(ng^2) compares, only for ng <= 256.
    for (int e = tid; e < ng; e += kThreads) {
      if (ng <= 256) {
        const int64_t ce = s_pre[e + 1] - s_pre[e];
        int rank = 0;
        for (int f = 0; f < ng; ++f) {
          const int64_t cf = s_pre[f + 1] - s_pre[f];
          rank += (cf > ce) || (cf == ce && f < e);
        }
        s_order[rank] = e;
      } else {
        s_order[e] = e;
      }
    }
    __syncthreads();
  }
}

// Banded order of a tiles_m x tiles_n tile grid: bands of kBand tile rows,
// column-major inside a band.  The 64 tiles an XCD runs at once (32 CUs x 2
// workgroups) then span 8 A row panels and 8 B column panels, which fit its
// 4 MB L2 together, and the A panels stay resident while the band sweeps N.
constexpr int kBand = 8;
__device__ __forceinline__ void band_tile(int64_t local, int64_t tiles_m, int64_t tiles_n,
                                          int64_t &tm, int64_t &tn) {
  const int64_t band = local / (kBand * tiles_n);
  const int64_t r = local - band * kBand * tiles_n;
  const int64_t left = tiles_m - band * kBand;
  const int rows = (int)(left < kBand ? left : kBand);
  const int64_t q = r / rows;
  tn = q;
  tm = band * kBand + (r - q * rows);
}

template <int GRID, int MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(4, 4))) void gemm_kernel(GemmArgs g) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  Stage *stages = reinterpret_cast<Stage *>(smem);
  int64_t *s_off = reinterpret_cast<int64_t *>(smem + 2 * sizeof(Stage));
  int64_t *s_pre = s_off + (kMaxGemmGroups + 1);
  int64_t *s_scan = s_pre + (kMaxGemmGroups + 1);
  int *s_order = reinterpret_cast<int *>(s_scan + kThreads);

  const int64_t tiles_m = (g.M + kBM - 1) / kBM;
  const int64_t tiles_n = (g.N + kBN - 1) / kBN;
  const int64_t kblocks = g.kpad / 16;
  if (MODE != 0) load_gemm_groups<MODE>(g, s_off, s_pre, s_scan, s_order);

  int64_t total;
  if (MODE == 0) total = tiles_m * tiles_n * g.n_split;
  else if (MODE == 1) total = s_pre[g.n_groups];
  else total = (int64_t)g.n_groups * tiles_m * tiles_n;
  // Dense and M-grouped tiles all cost the same K, so each XCD takes a
  // contiguous range of the tile order (L2 reuse of A and B panels): the
  // workgroups of XCD x (every kXcds-th one, as the dispatcher deals them out
  // round robin) stride through [x * per, (x + 1) * per).  K-grouped tiles
  // differ in cost by group, so they go round robin, heaviest group first.
  const int64_t slots = (int64_t)gridDim.x;
  const int64_t lanes = slots < kXcds ? slots : kXcds;
  const int64_t xcd = (MODE == 2) ? 0 : (int64_t)blockIdx.x % lanes;
  const int64_t per = (MODE == 2) ? total : (total + lanes - 1) / lanes;
  const int64_t t_end = min(xcd * per + per, total);
  const int64_t t_step = (MODE == 2) ? slots : (slots - xcd + lanes - 1) / lanes;
  const int64_t t_first = (MODE == 2) ? (int64_t)blockIdx.x
                                      : xcd * per + (int64_t)blockIdx.x / lanes;

  const int64_t t_end_s = wave_uniform(t_end);
  for (int64_t t = t_first;; t += t_step) {
    // Loop-invariant 64-bit operands of the tile bookkeeping, made opaque per
    // tile: the compares and the divisions below run on the vector unit, and
    // hoisting their VGPR copies out of the loop would keep them live (and
    // spilled) across the K loop.
    int64_t kblocks_t = kblocks, tiles_n_t = tiles_n, t_end_t = t_end_s;
    asm volatile("" : "+s"(kblocks_t), "+s"(tiles_n_t), "+s"(t_end_t));
    if (t >= t_end_t) break;
    TileJob job;
    if (MODE == 0) {
      // split-K: tile t of split s covers blocks [s * split_kb, ...) and
      // writes its partial sums at s * split_stride
      const int64_t tiles = tiles_m * tiles_n;
      int64_t sp = 0, local = t;
      while (local >= tiles) {   // at most kMaxSplits - 1 steps, no 64-bit division
        local -= tiles;
        ++sp;
      }
      int64_t tm, tn;
      band_tile(local, tiles_m, tiles_n_t, tm, tn);
      job.a_row0 = tm * kBM;
      job.a_rows = min((int64_t)kBM, g.M - job.a_row0);
      job.b_row0 = tn * kBN;
      job.b_rows = min((int64_t)kBN, g.N - job.b_row0);
      job.kb0 = min(sp * g.split_kb, kblocks_t);
      job.kb1 = min(job.kb0 + g.split_kb, kblocks_t);
      job.c_off = sp * g.split_stride + job.a_row0 * g.ldc + job.b_row0;
    } else if (MODE == 1) {
      int lo = 0, hi = g.n_groups;   // largest e with s_pre[e] <= t
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pre[mid] <= t) lo = mid; else hi = mid;
      }
      const int e = lo;
      const int64_t local = t - s_pre[e];
      int64_t tm, tn;
      band_tile(local, (s_pre[e + 1] - s_pre[e]) / tiles_n_t, tiles_n_t, tm, tn);
      job.a_row0 = s_off[e] + tm * kBM;
      job.a_rows = min((int64_t)kBM, s_off[e + 1] - job.a_row0);
      job.b_row0 = (int64_t)e * g.N + tn * kBN;
      job.b_rows = min((int64_t)kBN, g.N - tn * kBN);
      job.kb0 = 0;
      job.kb1 = kblocks;
      job.c_off = job.a_row0 * g.ldc + tn * kBN;
    } else {
      const int64_t per_group = tiles_m * tiles_n_t;
      const int64_t slot = t / per_group;
      const int64_t local = t - slot * per_group;
      const int64_t e = s_order[slot];
      const int64_t tm = local / tiles_n_t, tn = local - tm * tiles_n_t;
      job.a_row0 = tm * kBM;
      job.a_rows = min((int64_t)kBM, g.M - job.a_row0);
      job.b_row0 = tn * kBN;
      job.b_rows = min((int64_t)kBN, g.N - job.b_row0);
      job.kb0 = min(s_pre[e] / 16, kblocks_t);
      job.kb1 = min(s_pre[e + 1] / 16, kblocks_t);
      job.c_off = e * g.M * g.ldc + job.a_row0 * g.ldc + job.b_row0;
    }
    if (MODE != 0) {
      // the group tables come from LDS: keep the tile's (uniform) bounds in
      // scalar registers rather than in vector registers across the K loop
      job.a_row0 = wave_uniform(job.a_row0);
      job.a_rows = wave_uniform(job.a_rows);
      job.b_row0 = wave_uniform(job.b_row0);
      job.b_rows = wave_uniform(job.b_rows);
      job.kb0 = wave_uniform(job.kb0);
      job.kb1 = wave_uniform(job.kb1);
      job.c_off = wave_uniform(job.c_off);
    }
    Gemm<GRID> gm(g, job);
    gm.run(stages);
    __syncthreads();
  }
}

static size_t smem_bytes(int mode) {
  size_t b = 2 * sizeof(Stage);
  if (mode != 0)
    b += (2 * (kMaxGemmGroups + 1) + kThreads) * sizeof(int64_t) + kMaxGemmGroups * sizeof(int);
  return b;
}

template <int GRID, int MODE>
static hipError_t launch_t(const GemmArgs &g, int64_t blocks, hipStream_t st) {
  const size_t sm = smem_bytes(MODE);
  // The dynamic-LDS limit is a per-device function attribute: set it once on
  // each device the kernel runs on (a bit per device id; concurrent first
  // calls at worst both set it, which is harmless).
  static std::atomic<uint64_t> configured{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit == 0 || (configured.load(std::memory_order_acquire) & bit) == 0) {
    e = hipFuncSetAttribute((const void *)gemm_kernel<GRID, MODE>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sm);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_release);
  }
  hipLaunchKernelGGL((gemm_kernel<GRID, MODE>), dim3((unsigned)blocks), dim3(kThreads), sm, st, g);
  return hipGetLastError();
}

// Deterministic split-K sum: c[m, n] = sum over s = 0, 1, ... of the
// partial outputs ws[s][m][n] (FP32 adds in that fixed order).
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float *__restrict__ ws,
                                                         int n_split, int64_t M, int64_t N,
                                                         int64_t stride, float *__restrict__ c,
                                                         int64_t ldc) {
  const int64_t total = M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / N, n = i - m * N;
    float acc = ws[i];
    for (int sp = 1; sp < n_split; ++sp) acc += ws[sp * stride + i];
    __builtin_nontemporal_store(acc, c + m * ldc + n);
  }
}

int gemm_splits(int64_t M, int64_t N, int64_t kpad) {
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  int64_t s = kSplitSlots / (tiles > 0 ? tiles : 1);
  if (s > kMaxSplits) s = kMaxSplits;
  const int64_t by_k = (kpad / 16) / kMinSplitBlocks;
  if (s > by_k) s = by_k;
  return s >= 2 ? (int)s : 1;
}

hipError_t launch_gemm_split(const GemmArgs &g, float *ws, hipStream_t st) {
  GemmArgs p = g;
  const int64_t kblocks = g.kpad / 16;
  p.c = ws;
  p.ldc = g.N;
  p.out_bf16 = 0;
  p.split_kb = (kblocks + g.n_split - 1) / g.n_split;
  p.split_stride = g.M * g.N;
  hipError_t e = launch_gemm(p, st);
  if (e != hipSuccess) return e;
  int64_t blocks = (g.M * g.N + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, st, ws, g.n_split,
                     g.M, g.N, p.split_stride, static_cast<float *>(g.c), g.ldc);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &g, hipStream_t st) {
  const int64_t tiles_m = (g.M + kBM - 1) / kBM;
  const int64_t tiles_n = (g.N + kBN - 1) / kBN;
  int64_t total;
  if (g.mode == 0) total = tiles_m * tiles_n * g.n_split;
  else if (g.mode == 1) total = (tiles_m + g.n_groups) * tiles_n;   // upper bound
  else total = (int64_t)g.n_groups * tiles_m * tiles_n;
  int64_t blocks = total < 1 ? 1 : total;
  if (blocks > 65536) blocks = 65536;
#define UFP4_G(GR, MO) return launch_t<GR, MO>(g, blocks, st)
  if (g.grid == kGridUniform) {
    if (g.mode == 0) UFP4_G(kGridUniform, 0);
    if (g.mode == 1) UFP4_G(kGridUniform, 1);
    UFP4_G(kGridUniform, 2);
  }
  if (g.grid == kGridE2M1) {
    if (g.mode == 0) UFP4_G(kGridE2M1, 0);
    if (g.mode == 1) UFP4_G(kGridE2M1, 1);
    UFP4_G(kGridE2M1, 2);
  }
  if (g.mode == 0) UFP4_G(kGridE2M1Max2, 0);
  if (g.mode == 1) UFP4_G(kGridE2M1Max2, 1);
  UFP4_G(kGridE2M1Max2, 2);
#undef UFP4_G
}

}  // namespace ufp4
