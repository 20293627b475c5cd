// vif_kernels.hip -- HIP kernel of the float VIF feature for gfx950.
//
// One kernel per scale s does, for a 112 x 16 tile of output pixels:
//   1. stage the tile's input (+ halo of the filter radius) into LDS in the
//      plane's sample type, mirroring out-of-plane indices by one
//      reflection and a clamp (ADR-1444 "float_vif_hip runs the arithmetic
//      of the CUDA twin ...", Decision); samples are converted to fp32 where
//      they are read, and their normalisation (Research-2130 "float_ssim
//      decimation on the SYCL device", Sources: 8-bit as is, 10/12/16-bit
//      divided by 4/16/256) rides on the vertical pass's taps (VTaps);
//   2. the vertical pass of the separable Gaussian for the five quantities
//      x, y, x*x, y*y, x*y, one thread per column and plane with all 16 of
//      the tile's rows in registers (its plane's mean and square, half the
//      rows of the cross product), and the vertical pass of the next
//      scale's low-pass at even rows;
//   3. the horizontal pass (7 outputs per thread, in two rounds of
//      quantities so the block's LDS stays small), the per-pixel statistic
//      and the two terms, staged in LDS;
//   4. the horizontal pass of the next scale's low-pass at even columns,
//      written as the next scale's fp32 planes (2x decimation);
//   5. the ordered row sums themselves: each row's fp32 accumulator is
//      carried from tile to tile along the row (chain_rows), and the row's
//      last tile stores its sum; no term ever leaves the block.
//
// Every multiply and add is its own IEEE fp32 rounding (the library is
// built with -ffp-contract=off), taps in ascending order, vertical pass
// before horizontal.  A filter accumulator starts at its first product
// instead of 0.0f + product: every filter input is >= +0 (samples, their
// products and their low-passes), so the product is never -0 and the two
// are the same value.
#include <hip/hip_runtime.h>

#include <algorithm>

#include <type_traits>

#include "vif_device_math.h"
#include "vif_internal.h"

namespace vifk {

constexpr int kThreads = 256;

// Planes hold at most 2^27 samples, so a 32-bit offset addresses them.
// The input tile stays in LDS in the plane's own sample type (one byte per
// 8-bit sample); to_float converts a sample where the vertical pass reads
// it.  The pages normalise samples to fp32 (Research-2130 "float_ssim
// decimation on the SYCL device", Sources: 8-bit samples as they are, wider
// ones divided by 4, 16 or 256).  For 10- to 16-bit samples that division,
// by a power of two s, is carried by the vertical pass's taps instead (see
// VTaps): the pass then reads the samples as they are.
template <typename InT> __device__ __forceinline__ float to_float(InT v);

template <> __device__ __forceinline__ float to_float<uint8_t>(uint8_t v) {
  return static_cast<float>(v);
}

template <> __device__ __forceinline__ float to_float<uint16_t>(uint16_t v) {
  return static_cast<float>(v);
}

template <> __device__ __forceinline__ float to_float<float>(float v) {
  return v;
}

// Tap k of an n-tap filter.  The taps are symmetric bit for bit (t[k] and
// t[n-1-k] are the same fp32 value, checked on the host when the context is
// created), so the kernels read only t[min(k, n-1-k)]: the products
// t[k]*v and t[n-1-k]*v of the same sample are then one expression, which
// the compiler computes once.  Same values, fewer multiplies.
__device__ __forceinline__ float tap(const TapArgs &t, int k, int n) {
  return t.t[k < n - 1 - k ? k : n - 1 - k];
}

// Makes each value of v exist in a register at this point of the program.
// The empty asm takes the values as register operands, so the arithmetic
// that produces them cannot be moved below it (past a barrier, towards its
// later use), which would keep its many inputs live instead of the few
// results.  It emits no instruction.
template <int A, int B>
__device__ __forceinline__ void settle(float (&v)[A][B]) {
#pragma unroll
  for (int a = 0; a < A; ++a)
#pragma unroll
    for (int b = 0; b < B; ++b)
      asm volatile("" : "+v"(v[a][b]));
}

// An LDS float index the compiler treats as unknown.  Accesses at constant
// distances from it then share one address register and carry the
// distances in their instructions' offset fields.  Otherwise the compiler
// folds a block-uniform part above the paired read's 8-bit offset range into
// each address and spends a vector add per pair.  The value is unchanged.
__device__ __forceinline__ int lds_base(int i) {
  asm volatile("" : "+v"(i));
  return i;
}

// LDS layout of the vertical results (bank = dword address mod 64 for a
// whole wave, or mod 32 for each half of it; the layouts below avoid
// conflicts in both readings).
//
// Rows of the five quantities: pitch vpitch(R), the smallest pitch >= the
// vertical pass's CW = kTileW + 2R columns that is 8 mod 16.  The horizontal
// pass reads with lane l of a wave at row (l >> 3) + 8a and column
// 7 * ((l & 7) + 8b) + j: the 8 lanes of a row read 8 columns 7 apart, and
// rows 8 (mod 16) dwords apart move those 8 banks to 8 disjoint sets, so
// the 64 lanes (and each half's 32) hit distinct banks.
template <int R>
__host__ __device__ constexpr int vpitch() {
  return kTileW + 2 * R + ((8 - (kTileW + 2 * R)) % 16 + 16) % 16;
}

// Rows of the next scale's vertical low-pass (8 rows per plane): row yd
// starts at dec_row(yd), which is (yd & 3) + 32 * (yd >> 2) mod 64, and a
// plane takes kDecPlane floats.  The decimation reads with lane l at row
// (l >> 3) & 7 and columns 4 * (l & 7) + c apart: the 8 columns of a row lie
// 4 apart, and the rows' start residues (0..3 and 32..35) interleave them.
__device__ __forceinline__ int dec_row(int yd) {
  return 128 * yd + (yd & 3) + 32 * (yd >> 2);
}
constexpr int kDecPlane = 1088; // >= dec_row(7) + 128, 0 mod 64

// Input row j (counted from the first input row the outputs read) of one
// quantity into the vertical accumulators a[i] of OUT consecutive output
// rows: output i adds tap j - i; its first tap starts the accumulator.
template <int N, int OUT>
__device__ __forceinline__ void vacc(float (&a)[OUT], float val, int j, int,
                                     const TapArgs &taps) {
#pragma unroll
  for (int i = 0; i < OUT; ++i) {
    const int k = j - i;
    if (k >= 0 && k < N) {
      const float t = tap(taps, k, N);
      a[i] = k == 0 ? t * val : a[i] + t * val;
    }
  }
}

template <int A>
__device__ __forceinline__ void settle1(float (&v)[A]) {
#pragma unroll
  for (int a = 0; a < A; ++a)
    asm volatile("" : "+v"(v[a]));
}

// The vertical pass's taps: m for the planes' means, q for their squares
// and the cross product, d for the next scale's low-pass.  Normally m and q
// are the scale's taps t and d the next scale's, dt.  For 10- to 16-bit
// samples v, normalised as v * s with s = 2^-2, 2^-4 or 2^-8, they are t *
// s, t * s^2 and dt * s (exact: powers of two times normal fp32 values) and
// the pass reads v itself, with the same fp32 results: t * (v * s) and
// (t * s) * v are one real number rounded once; (v * s)^2 rounds to fl(v^2)
// * s^2, a power-of-two scaling commuting with rounding (the values stay
// far from underflow and overflow), so t * fl((v * s)^2) and (t * s^2) *
// fl(v^2) are again one real number, and likewise for x * y and the
// low-pass; every sum then adds the same values.  That saves the multiply
// by s for each of the 56 samples a thread reads per tile.
struct VTaps {
  TapArgs m, q, d;
};

// The vertical pass of group G over a column of the input tile: so is the
// group's own plane, sp the other.  Own plane: mean vm and square vs at all
// kTileH rows, the next scale's low-pass vd at the even rows; cross product
// x*y: vx at rows G*kTileH/2 .. + kTileH/2 - 1, which read input rows from
// G*kTileH/2 on.  G is a template argument, so every tap index is a constant.
template <int R, int RD, typename InT, int G>
__device__ __forceinline__ void
vpass(const InT *so, const InT *sp, const TapArgs &tm, const TapArgs &tq,
      const TapArgs &dtaps, float (&vm)[kTileH], float (&vs)[kTileH],
      float (&vx)[kTileH / 2], float (&vd)[kTileH / 2]) {
  constexpr int N = 2 * R + 1;
  constexpr int ND = 2 * RD + 1;
  constexpr int CW = kTileW + 2 * R;
  constexpr int VR = kTileH;
  constexpr int VC = kTileH / 2;
#pragma unroll
  for (int j = 0; j < VR + 2 * R; ++j) {
    const float p = to_float<InT>(so[j * CW]);
    vacc<N, VR>(vm, p, j, 0, tm);
    vacc<N, VR>(vs, p * p, j, 0, tq);
    constexpr int J0 = G * VC;
    if (j >= J0 && j < J0 + VC + 2 * R) {
      const float o = to_float<InT>(sp[j * CW]);
      // x * y in that operand order whichever plane is the thread's own
      vacc<N, VC>(vx, G == 0 ? p * o : o * p, j - J0, 0, tq);
    }
    if constexpr (RD > 0) {
#pragma unroll
      for (int m = 0; m < VC; ++m) {
        const int k = j - 2 * m - R + RD;
        if (k >= 0 && k < ND) {
          const float t = tap(dtaps, k, ND);
          vd[m] = k == 0 ? t * p : vd[m] + t * p;
        }
      }
    }
  }
}

// Horizontal pass of NQ quantities stored in LDS as [q][kTileH][vpitch]:
// thread (ty, seg) computes tile row ty, columns seg*HB .. seg*HB+HB-1.
template <int R, int NQ, int HB>
__device__ __forceinline__ void hpass(const float *__restrict__ sV, int ty,
                                      int seg, const TapArgs &taps,
                                      float (&f)[NQ][HB]) {
  constexpr int N = 2 * R + 1;
  constexpr int CWP = vpitch<R>();
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const float *row = sV + lds_base((q * kTileH + ty) * CWP + seg * HB);
    float v[HB + 2 * R];
#pragma unroll
    for (int j = 0; j < HB + 2 * R; ++j)
      v[j] = row[j];
#pragma unroll
    for (int i = 0; i < HB; ++i) {
      float a = tap(taps, 0, N) * v[i];
#pragma unroll
      for (int k = 1; k < N; ++k)
        a = a + tap(taps, k, N) * v[i + k];
      f[q][i] = a;
    }
    // one quantity's row at a time: keeps the next row's loads from being
    // hoisted here, which would hold them all in registers at once
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Row sums carried from tile to tile.  The sum of a
// row is one fp32 accumulator over its terms from left to right (ADR-1422
// "float_vif_sycl computes the CPU's arithmetic ...", Context and Decision),
// so a row that spans several tiles is a chain: tile tx continues the
// accumulator that tile tx - 1 ended with.  Tile tx - 1 hands it over in one
// 64-bit word per sequence, io.carry[((z * strips + strip) * (ntx - 1) +
// tx - 1) * 32 + q]: the launch's tag in the high half, the fp32 value in the
// low half, written and read with relaxed atomics at device scope.  A word
// carrying the value with its tag needs no fence: a reader that sees the tag
// sees the value of the same store.  Words of an earlier launch carry an
// earlier tag, so they are never taken for this launch's.
//
// Blocks of a launch take the same tile column of every strip and frame
// before the next column (blockIdx.x runs over strips and frames), and the
// hardware starts blocks in that order, so tile tx - 1 started long before
// tile tx (a whole column of blocks earlier) and its word is usually there
// when tile tx reads it.  The wait is bounded: after kCarrySpins reads
// without the tag the block gives up, stores NaN and raises io.err, which
// the host reports as an error, so a launch always ends.
constexpr int kCarrySpins = 1 << 16;

__device__ __forceinline__ float wait_carry(const unsigned long long *word,
                                            unsigned tag, int *err) {
  unsigned long long v =
      __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  int spins = 0;
  while (static_cast<unsigned>(v >> 32) != tag) {
    if (++spins >= kCarrySpins) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      return __builtin_nanf("");
    }
    __builtin_amdgcn_s_sleep(2);
    v = __hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return __uint_as_float(static_cast<unsigned>(v));
}

// Lane q's part of the chain for tile (tx, strip) of frame z: `terms` is
// its sequence's row of the tile in LDS, `cols` the tile's columns inside
// the plane, y the sequence's row.
__device__ __forceinline__ void chain_rows(const ScaleIO &io,
                                           const float *__restrict__ terms,
                                           int cols, int z, int strip, int tx,
                                           int y, int h, int q) {
  unsigned long long *word =
      io.carry +
      ((static_cast<size_t>(z) * io.strips + strip) * (io.ntx - 1) + tx) *
          kSeq +
      q;
  float acc = 0.0f;
  if (tx > 0)
    acc = wait_carry(word - kSeq, io.carry_tag, io.err);
  if (cols == kTileW) {
#pragma unroll 16
    for (int i = 0; i < kTileW; ++i)
      acc = acc + terms[i];
  } else {
    for (int i = 0; i < cols; ++i)
      acc = acc + terms[i];
  }
  if (tx == io.ntx - 1) {
    if (y < h)
      io.rows[static_cast<size_t>(z) * io.rows_stride + 2 * y + (q & 1)] = acc;
  } else {
    const unsigned long long v =
        (static_cast<unsigned long long>(io.carry_tag) << 32) |
        __float_as_uint(acc);
    __hip_atomic_store(word, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The slot of this block in the grid's x dimension, in the XCD-aware order:
// block x runs on XCD x % 8 (the dispatcher deals the blocks of a launch
// round-robin over the eight XCDs, and gridDim.x is a multiple of 8), so
// slot (x % 8) * (gridDim.x / 8) + x / 8 gives each XCD a run of
// consecutive strips (which share halo rows in its L2), and the same strip
// of the next tile column lands on the same XCD.  Slots at or past the
// launch's frames x strips are padding.
__device__ __forceinline__ int block_slot() {
  const int per = static_cast<int>(gridDim.x) >> 3;
  return static_cast<int>(blockIdx.x & 7) * per +
         static_cast<int>(blockIdx.x >> 3);
}

// Step 1 of the scale kernels: the input tile [IR][CW] of ref, then of
// dist, into LDS in the planes' own sample type, for the tile whose first
// output pixel is (x0, y0).  A tile whose columns all lie inside the plane,
// in a plane that allows it (vec_in), loads 8 samples per thread and load:
// 16 threads per row, 16 rows per pass, two passes per plane (x0 - R is a
// multiple of 8, so every load is aligned).  Other tiles load one sample per
// thread and row, mirroring each column: waves 0-1 the even rows, waves 2-3
// the odd ones, so the row (and its mirror) is uniform in a wave.  Either way
// all of a thread's loads are issued before the first store.
template <int R, typename InT>
__device__ __forceinline__ void stage_tile(InT *sIn,
                                           const InT *__restrict__ ref,
                                           const InT *__restrict__ dist,
                                           int vec_in, int x0, int y0, int w,
                                           int h, int tid) {
  constexpr int CW = kTileW + 2 * R;
  constexpr int IR = kTileH + 2 * R;
  bool vec = false;
  if constexpr (sizeof(InT) < 4)
    vec = vec_in != 0 && x0 - R >= 0 && x0 - R + CW <= w;
  if (vec) {
    if constexpr (sizeof(InT) < 4) {
      constexpr int kSpl = 8;               // samples per load
      constexpr int kTpr = CW / kSpl;       // threads per row
      constexpr int kRpp = kThreads / kTpr; // rows per pass
      using Vec =
          typename std::conditional<sizeof(InT) == 1, uint2, uint4>::type;
      static_assert(sizeof(Vec) == kSpl * sizeof(InT), "8 samples");
      static_assert(CW % kSpl == 0 && IR % kRpp == 0, "whole passes");
      const int q = tid % kTpr;
      const int r0 = tid / kTpr;
      Vec a[IR / kRpp], b[IR / kRpp];
#pragma unroll
      for (int it = 0; it < IR / kRpp; ++it) {
        const int j = r0 + kRpp * it;
        const unsigned gy = static_cast<unsigned>(mirror_clamp(y0 - R + j, h));
        const unsigned base = gy * static_cast<unsigned>(w) + (x0 - R);
        a[it] = reinterpret_cast<const Vec *>(ref + base)[q];
        b[it] = reinterpret_cast<const Vec *>(dist + base)[q];
      }
#pragma unroll
      for (int it = 0; it < IR / kRpp; ++it) {
        const int j = r0 + kRpp * it;
        *reinterpret_cast<Vec *>(sIn + j * CW + kSpl * q) = a[it];
        *reinterpret_cast<Vec *>(sIn + IR * CW + j * CW + kSpl * q) = b[it];
      }
    }
  } else {
    const int c = tid & 127;
    const int half = __builtin_amdgcn_readfirstlane(tid >> 7);
    static_assert(IR % 2 == 0, "the two row phases cover the tile");
    if (c < CW) {
      const unsigned gx = static_cast<unsigned>(mirror_clamp(x0 - R + c, w));
#pragma unroll
      for (int it = 0; it < IR / 2; ++it) {
        const int j = half + 2 * it;
        const unsigned gy = static_cast<unsigned>(mirror_clamp(y0 - R + j, h));
        const unsigned off = gy * static_cast<unsigned>(w) + gx;
        sIn[j * CW + c] = ref[off];
        sIn[IR * CW + j * CW + c] = dist[off];
      }
    }
  }
}

// R: filter radius of this scale (taps 2R+1).  RD: radius of the next
// scale's low-pass (0 at the last scale: no decimation).
//
// LDS is reused phase by phase so that a block needs at most 25.5 KiB (six
// blocks per CU):
//   phases 1-2  input tile, native samples       [2][IR][CW] InT
//   phases 3-4  vertical results of x, y         [2][kTileH][vpitch]
//               + the low-pass at even rows      [2][kDecPlane] (dec_row)
//   phases 5-6  vertical results of x*x, y*y, x*y [3][kTileH][vpitch]
//   phases 7-8  terms                            [kSeq][kTermPitch]
// The horizontal pass therefore runs in two rounds (x, y and the next
// scale's planes, then the three second moments); the second round's
// vertical results wait in registers until its write.
//
// Tile (tx, strip) of frame z: blockIdx.x runs fastest over the strips of
// every frame (in the XCD-aware order of block_slot; gridDim.x is padded to a
// multiple of 8 and the padding blocks exit at once), so consecutive blocks
// take the same tile column of every strip and frame, and tx = first +
// blockIdx.y (a plane wider than a grid's y dimension allows is covered by
// several launches).  Frame z reads io.in_ref[z], io.in_dist[z] and writes
// at its own offsets of the next scale's planes and the row sums.
template <int R, int RD, typename InT, bool kPow2>
__global__ __launch_bounds__(kThreads) void scale_kernel(
    ScaleIO io, int w, int h, VTaps vt, TapArgs taps, TapArgs dtaps,
    StatArgs stat, int first) {
  const int sp = block_slot();
  if (sp >= io.slots)
    return; // padding block
  const int z = sp / io.strips;
  const int strip = sp - z * io.strips;
  const int tx = first + static_cast<int>(blockIdx.y);
  const InT *__restrict__ ref = static_cast<const InT *>(io.in_ref[z]);
  const InT *__restrict__ dist = static_cast<const InT *>(io.in_dist[z]);
  float *__restrict__ next_ref = io.next_ref + z * io.next_stride;
  float *__restrict__ next_dist = io.next_dist + z * io.next_stride;
  constexpr int N = 2 * R + 1;
  constexpr int ND = 2 * RD + 1;
  constexpr int CW = kTileW + 2 * R; // columns of the vertical pass
  constexpr int IR = kTileH + 2 * R; // input rows
  constexpr int CWP = vpitch<R>();   // conflict-free horizontal reads
  constexpr int HB = 7;              // outputs per thread, horizontal pass
  constexpr int kQA = 2;             // quantities of the first round
  constexpr int kInFloats =
      (2 * IR * CW * static_cast<int>(sizeof(InT)) + 3) / 4;
  constexpr int kVd = RD > 0 ? 2 * kDecPlane : 0;
  constexpr int kVA = kQA * kTileH * CWP + kVd;
  constexpr int kVB = (5 - kQA) * kTileH * CWP;
  constexpr int kT = kSeq * kTermPitch;
  constexpr int kL0 = kVA > kVB ? kVA : kVB;
  constexpr int kL1 = kL0 > kT ? kL0 : kT;
  constexpr int kLds = kL1 > kInFloats ? kL1 : kInFloats;
  static_assert(CW <= 128, "one thread per vertical column in two halves");
  static_assert(CWP >= CW && CWP % 16 == 8, "vertical-result pitch");
  static_assert(kTileH / 2 == 8 && kTileW / 4 <= 32, "decimation rows");
  static_assert(kTileW == 16 * HB, "16 horizontal segments per row");
  __shared__ __attribute__((aligned(16))) float lds[kLds];
  InT *sIn = reinterpret_cast<InT *>(lds);

  const int tid = threadIdx.x;
  const int x0 = tx * kTileW;
  const int y0 = strip * kTileH;
  // 1. input tile
  stage_tile<R, InT>(sIn, ref, dist, io.vec_in, x0, y0, w, h, tid);
  __syncthreads();

  // 2. vertical passes: thread (vc, g) owns column vc and one plane, g = 0
  //    (waves 0-1) ref, g = 1 (waves 2-3) dist: the plane's mean and square
  //    at all kTileH rows, the next scale's low-pass of the plane at the even
  //    rows, and the cross product x*y at rows 8g .. 8g + 7.  Owning every
  //    row of a column, a thread reads each input row once and shares more of
  //    the symmetric taps' products between its outputs; the two groups do
  //    the same work and keep the same registers.
  constexpr int VR = kTileH;
  constexpr int VC = kTileH / 2;       // rows of the cross product per group
  const int vc = tid & 127;
  const int vg = __builtin_amdgcn_readfirstlane(tid >> 7);
  const bool vact = vc < CW;
  float vm[VR], vs[VR], vx[VC], vd[VC];
  if (vact) {
    const InT *so = sIn + vg * IR * CW + vc;       // own plane
    const InT *sp = sIn + (1 - vg) * IR * CW + vc; // the other plane
    // the taps with the samples' normalisation for 10- to 16-bit planes
    constexpr bool kScaled = std::is_same<InT, uint16_t>::value;
    const TapArgs &tm = kScaled ? vt.m : taps;
    const TapArgs &tq = kScaled ? vt.q : taps;
    const TapArgs &td = kScaled ? vt.d : dtaps;
    if (vg == 0)
      vpass<R, RD, InT, 0>(so, sp, tm, tq, td, vm, vs, vx, vd);
    else
      vpass<R, RD, InT, 1>(so, sp, tm, tq, td, vm, vs, vx, vd);
    settle1(vm);
    settle1(vs);
    settle1(vx);
    if constexpr (RD > 0)
      settle1(vd);
  }
  __syncthreads(); // the input tile is dead from here on

  float *sV = lds;
  float *sVd = lds + kQA * kTileH * CWP;
  // horizontal pass: wave w takes tile rows 8 * (w & 1) .. + 7 and segments
  // 8 * (w >> 1) .. + 7; lane l row l >> 3, segment l & 7 (see vpitch)
  const int seg = (tid & 7) + 8 * (tid >> 7);
  const int ty = ((tid >> 3) & 7) + 8 * ((tid >> 6) & 1);

  // 3. round A: vertical results of x (group 0) and y (group 1), and each
  //    plane's vertical low-pass, to LDS
  if (vact) {
#pragma unroll
    for (int i = 0; i < VR; ++i)
      sV[(vg * kTileH + i) * CWP + vc] = vm[i];
    if constexpr (RD > 0) {
#pragma unroll
      for (int m = 0; m < VC; ++m)
        sVd[vg * kDecPlane + dec_row(m) + vc] = vd[m];
    }
  }
  __syncthreads();

  // 4. horizontal pass of x, y: thread (ty, seg) owns tile row ty and
  //    columns seg*7 .. seg*7+6.
  float fa[kQA][HB];
  hpass<R, kQA, HB>(sV, ty, seg, taps, fa);
  settle(fa);

  //    next scale's planes: horizontal low-pass at even columns of the even
  //    rows.  Thread (yd, sd) owns decimated row yd and columns 2sd, 2sd+1;
  //    wave w takes sd = 8w .. 8w + 7, lane l row (l >> 3) & 7 and
  //    sd = 8w + (l & 7) (see dec_row).
  if constexpr (RD > 0) {
    const int sd = (tid & 7) + 8 * (tid >> 6);
    const int yd = (tid >> 3) & 7;
    const int wd = w >> 1;
    const int hd = h >> 1;
    const int ydg = (y0 >> 1) + yd;
    if (sd < kTileW / 4 && ydg < hd) {
      const float *drow[2];
#pragma unroll
      for (int p = 0; p < 2; ++p)
        drow[p] = lds + lds_base(static_cast<int>(sVd - lds) + p * kDecPlane +
                                 dec_row(yd) + 4 * sd + R - RD);
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        const int xl = sd * 2 + o;
        const int xdg = (x0 >> 1) + xl;
        if (xdg < wd) {
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const float *row = drow[p] + 2 * o;
            float a = tap(dtaps, 0, ND) * row[0];
#pragma unroll
            for (int k = 1; k < ND; ++k)
              a = a + tap(dtaps, k, ND) * row[k];
            float *dst = p == 0 ? next_ref : next_dist;
            dst[static_cast<size_t>(ydg) * wd + xdg] = a;
          }
        }
      }
    }
  }
  __syncthreads(); // round A's region is free

  // 5. round B: vertical results of x*x (group 0), y*y (group 1) and x*y
  //    (rows 8g .. 8g + 7) to LDS
  if (vact) {
#pragma unroll
    for (int i = 0; i < VR; ++i)
      sV[(vg * kTileH + i) * CWP + vc] = vs[i];
#pragma unroll
    for (int i = 0; i < VC; ++i)
      sV[(2 * kTileH + vg * VC + i) * CWP + vc] = vx[i];
  }
  __syncthreads();

  // 6. horizontal pass of x*x, y*y, x*y, then the statistic; the terms stay
  //    in registers
  float tnum[HB], tden[HB];
  {
    float fb[5 - kQA][HB];
    hpass<R, 5 - kQA, HB>(sV, ty, seg, taps, fb);
    settle(fb);
#pragma unroll
    for (int i = 0; i < HB; ++i)
      pixel_terms<kPow2>(fa[0][i], fa[1][i], fb[0][i], fb[1][i], fb[2][i],
                         stat, tnum[i], tden[i]);
  }
  __syncthreads(); // every read of round B is done: its region takes the terms

  // 7. terms to LDS as 32 sequences (row-major per row and component):
  //    sT[2*ty + c][x], the order in which the row sums read them.
  float *sT = lds;
#pragma unroll
  for (int i = 0; i < HB; ++i) {
    sT[(2 * ty) * kTermPitch + seg * HB + i] = tnum[i];
    sT[(2 * ty + 1) * kTermPitch + seg * HB + i] = tden[i];
  }
  __syncthreads(); // terms complete in LDS

  // 8. the ordered row sums, continued from the tile on the left: lane q of
  //    wave 0 owns sequence q (row q / 2, component q % 2); it takes the
  //    row's fp32 accumulator where the left tile left it (0 at the first
  //    tile), adds this tile's terms left to right, and hands the
  //    accumulator on, or stores the row's sum at the last tile.
  if (tid < kSeq)
    chain_rows(io, sT + tid * kTermPitch, min(kTileW, w - x0), z, strip, tx,
               y0 + (tid >> 1), h, tid);
}

// ------------------------------------------------------------ staging probe

// Scale 0's input staging alone: the blocks of a scale-0 launch, in the same
// order and with the scale kernel's own staging code, load the same tiles
// into LDS and do nothing else; each block then adds its tile's samples and
// stores the sum at out[tx * slots + slot], so no load is dead and the host
// can check what was read.  Its fetched bytes, against the lines its blocks
// touch, calibrate the HBM traffic counters for the scale kernel's access
// shape.
template <typename InT>
__global__ __launch_bounds__(kThreads) void stage_probe_kernel(
    ScaleIO io, int w, int h, int first, unsigned *__restrict__ out) {
  constexpr int R = 8;
  constexpr int kElems = 2 * (kTileH + 2 * R) * (kTileW + 2 * R);
  __shared__ __attribute__((aligned(16))) InT sIn[kElems];
  __shared__ unsigned red[kThreads / 64];
  const int sp = block_slot();
  if (sp >= io.slots)
    return; // padding block
  const int z = sp / io.strips;
  const int strip = sp - z * io.strips;
  const int tx = first + static_cast<int>(blockIdx.y);
  const int tid = threadIdx.x;
  stage_tile<R, InT>(sIn, static_cast<const InT *>(io.in_ref[z]),
                     static_cast<const InT *>(io.in_dist[z]), io.vec_in,
                     tx * kTileW, strip * kTileH, w, h, tid);
  __syncthreads();
  unsigned sum = 0;
  for (int i = tid; i < kElems; i += kThreads)
    sum += sIn[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1)
    sum += __shfl_down(sum, off);
  if ((tid & 63) == 0)
    red[tid >> 6] = sum;
  __syncthreads();
  if (tid == 0)
    out[static_cast<size_t>(tx) * io.slots + sp] =
        red[0] + red[1] + red[2] + red[3];
}

// ------------------------------------------------------------------ launch

// One launch of the scale kernel of `scale` for the statistic's form kPow2
// (a power-of-two noise variance, see den_ratio).
template <bool kPow2>
void launch_one(int scale, int bpc, dim3 grid, dim3 block, hipStream_t stream,
                const ScaleIO &io, const ScaleGeom &g, float sc,
                const TapArgs &taps, const TapArgs &next_taps,
                const StatArgs &stat, int first) {
  VTaps vt{}; // read by the 10- to 16-bit scale-0 kernels only
  switch (scale) {
  case 0:
    if (bpc == 8) {
      scale_kernel<8, 4, uint8_t, kPow2><<<grid, block, 0, stream>>>(
          io, g.w, g.h, vt, taps, next_taps, stat, first);
    } else {
      // sc is 2^-2, 2^-4 or 2^-8: every product below is exact
      for (int k = 0; k < kMaxTaps; ++k) {
        vt.m.t[k] = taps.t[k] * sc;
        vt.q.t[k] = taps.t[k] * sc * sc;
        vt.d.t[k] = next_taps.t[k] * sc;
      }
      scale_kernel<8, 4, uint16_t, kPow2><<<grid, block, 0, stream>>>(
          io, g.w, g.h, vt, taps, next_taps, stat, first);
    }
    break;
  case 1:
    scale_kernel<4, 2, float, kPow2><<<grid, block, 0, stream>>>(
        io, g.w, g.h, vt, taps, next_taps, stat, first);
    break;
  case 2:
    scale_kernel<2, 1, float, kPow2><<<grid, block, 0, stream>>>(
        io, g.w, g.h, vt, taps, next_taps, stat, first);
    break;
  default:
    scale_kernel<1, 0, float, kPow2><<<grid, block, 0, stream>>>(
        io, g.w, g.h, vt, taps, next_taps, stat, first);
    break;
  }
}

hipError_t launch_scale(int scale, int bpc, const ScaleIO &io, int n,
                        const ScaleGeom &g, const TapArgs &taps,
                        const TapArgs &next_taps, const StatArgs &stat,
                        hipStream_t stream) {
  if (n < 1 || n > kMaxBatch || scale < 0 || scale > 3)
    return hipErrorInvalidValue;
  const dim3 block(kThreads);
  const float sc = bpc == 8    ? 1.0f
                   : bpc == 10 ? 0.25f
                   : bpc == 12 ? 0.0625f
                               : 0.00390625f;
  // Grid x runs over the strips of every frame, grid y over the tile
  // columns, at most kMaxGridY per launch.  A later launch on the same
  // stream starts after the earlier ones have finished, so a chain that
  // crosses launches finds its carries written.
  if (io.carry == nullptr || io.rows == nullptr || io.err == nullptr ||
      io.strips != g.strips || io.ntx != g.ntx ||
      static_cast<long>(n) * g.strips > 0x7ffffff8L) // padded grid x fits
    return hipErrorInvalidValue;
  ScaleIO iox = io;
  iox.slots = n * g.strips;
  for (int first = 0; first < g.ntx; first += kMaxGridY) {
    const dim3 grid(static_cast<unsigned>((n * g.strips + 7) & ~7),
                    static_cast<unsigned>(std::min(kMaxGridY, g.ntx - first)),
                    1);
    if (stat.inv_nsq != 0.0)
      launch_one<true>(scale, bpc, grid, block, stream, iox, g, sc, taps,
                       next_taps, stat, first);
    else
      launch_one<false>(scale, bpc, grid, block, stream, iox, g, sc, taps,
                        next_taps, stat, first);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return e;
  }
  return hipSuccess;
}

hipError_t launch_scale0_column(const ScaleIO &io, const ScaleGeom &g,
                                const TapArgs &taps, const TapArgs &next_taps,
                                const StatArgs &stat, int col,
                                hipStream_t stream) {
  if (col < 0 || col >= g.ntx || io.carry == nullptr || io.rows == nullptr ||
      io.err == nullptr || io.strips != g.strips || io.ntx != g.ntx)
    return hipErrorInvalidValue;
  ScaleIO iox = io;
  iox.slots = g.strips;
  const dim3 grid(static_cast<unsigned>((g.strips + 7) & ~7), 1, 1);
  if (stat.inv_nsq != 0.0)
    scale_kernel<8, 4, uint8_t, true><<<grid, dim3(kThreads), 0, stream>>>(
        iox, g.w, g.h, VTaps{}, taps, next_taps, stat, col);
  else
    scale_kernel<8, 4, uint8_t, false><<<grid, dim3(kThreads), 0, stream>>>(
        iox, g.w, g.h, VTaps{}, taps, next_taps, stat, col);
  return hipGetLastError();
}

hipError_t launch_stage_probe(int bpc, const ScaleIO &io, int n,
                              const ScaleGeom &g, unsigned *out,
                              hipStream_t stream) {
  if (n < 1 || n > kMaxBatch || out == nullptr || io.strips != g.strips ||
      io.ntx != g.ntx)
    return hipErrorInvalidValue;
  ScaleIO iox = io;
  iox.slots = n * g.strips;
  for (int first = 0; first < g.ntx; first += kMaxGridY) {
    const dim3 grid(static_cast<unsigned>((n * g.strips + 7) & ~7),
                    static_cast<unsigned>(std::min(kMaxGridY, g.ntx - first)),
                    1);
    if (bpc == 8)
      stage_probe_kernel<uint8_t><<<grid, dim3(kThreads), 0, stream>>>(
          iox, g.w, g.h, first, out);
    else
      stage_probe_kernel<uint16_t><<<grid, dim3(kThreads), 0, stream>>>(
          iox, g.w, g.h, first, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return e;
  }
  return hipSuccess;
}

hipError_t scale0_resident_blocks(int bpc, int *blocks) {
  int per_cu = 0;
  hipError_t e =
      bpc == 8 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                     &per_cu, scale_kernel<8, 4, uint8_t, true>, kThreads, 0)
               : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                     &per_cu, scale_kernel<8, 4, uint16_t, true>, kThreads,
                     0);
  int dev = 0, cus = 0;
  if (e == hipSuccess)
    e = hipGetDevice(&dev);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount,
                              dev);
  *blocks = per_cu * cus;
  return e;
}

} // namespace vifk
