// vif_internal.h -- host-side declarations shared by the library's
// translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

struct vif_options; // include/vif.h

namespace vifk {

constexpr int kScales = 4;
constexpr int kMaxTaps = 17;
constexpr int kWidths[kScales] = {17, 9, 5, 3};

// Tile of the per-scale kernel: 112 output columns x 16 output rows, and
// the row strip of the term layout (16 rows).
constexpr int kTileW = 112;
constexpr int kTileH = 16;

struct TapArgs {
  float t[kMaxTaps];
};

// Constants of the per-pixel statistic, built on the host from the options
// and passed to every scale kernel by value.
//   nsq      the noise variance (a double, as the branch and both ratios
//            use it)
//   inv_nsq  1 / nsq when that is a power of two in [2^-20, 2^20], so that
//            s * inv_nsq is the quotient s / nsq exactly; 0 otherwise
//            (divide).  Non-zero selects the kernels' kPow2 form.
//   nsq_f, inv_nsq_f  nsq and inv_nsq as fp32 values when inv_nsq is not
//            0 (both are then powers of two in [2^-20, 2^20], exact in
//            fp32); 0 otherwise
//   gain     the enhancement gain limit rounded to fp32.  C's MIN(g, limit)
//            with a double limit selects the same value as the fp32
//            comparison g < gain: no fp32 value lies strictly between a
//            limit and its nearest fp32, so the two comparisons can differ
//            only where g is that fp32 value, and then both results are g.
struct StatArgs {
  double nsq;
  double inv_nsq;
  float gain;
  float nsq_f;
  float inv_nsq_f;
};

// Option checks and the statistic constants (vif_options.cpp).  Returns
// false for options outside their documented ranges.
struct OptionValues {
  double sigma_nsq, enhn_gain_limit, kernelscale, scale_min_val[3];
  int skip_scale0;
};
bool options_valid(const OptionValues &o);
StatArgs make_stat_args(double nsq, double gain_limit);

// Terms of a 16-row strip: 32 sequences (16 rows x {num, den}).  In LDS a
// tile keeps them as [seq][x] with pitch kTermPitch; an odd pitch puts the
// 32 sequences' same column in 32 different banks, so the lanes that read
// one sequence each (the row sums) never share a bank.
constexpr int kSeq = 32;
constexpr int kTermPitch = kTileW + 1;

// Frames one launch may carry (grid x of the scale kernels runs over the
// strips of every frame).
constexpr int kMaxBatch = 16;
// Blocks per launch in grid dimension y (the runtime allows 65536; a plane
// with more columns of tiles takes several launches).
constexpr int kMaxGridY = 65535;

// Inputs and outputs of one launch of a scale kernel for n frames: frame z
// reads in_ref[z] / in_dist[z] (the caller's frames at scale 0, the
// context's planes above) and writes the next scale's planes at next_* + z *
// next_stride (floats) and its rows' sums at rows[z * rows_stride + 2 * y +
// c] (c = 0 for the numerator, 1 for the denominator).  Each row's sum is
// carried from tile to tile in carry: n * strips * (ntx - 1) * 32 words (at
// least 32), written with the tag carry_tag (never 0, new for every launch
// that reuses the words); err is raised if a wait for a word gives up.
// strips and ntx are the scale's.
struct ScaleIO {
  const void *in_ref[kMaxBatch];
  const void *in_dist[kMaxBatch];
  float *next_ref;
  float *next_dist;
  size_t next_stride;
  // scale 0: every in_ref/in_dist plane may be read 8 samples per load
  // (width a multiple of 8, planes 8-byte aligned for 8-bit samples,
  // 16-byte for 16-bit ones); 0 otherwise and at scales 1-3
  int vec_in;
  unsigned long long *carry;
  unsigned carry_tag;
  int strips, ntx;
  int slots; // frames x strips: the grid's x dimension before its padding
  float *rows;
  size_t rows_stride;
  int *err;
};

// Host arithmetic on row sums (vif_rows.cpp).  scores_from_rows: rows
// holds nrows[s] pairs (n_y, d_y) for scale 0, then scale 1, ...; writes
// out[8] and the eight fp32 sums as the context's collect does.
void scores_from_rows(const float *rows, const int nrows[kScales],
                      const vif_options &opt, double out[8], float sums[8]);
// out[8] from the eight fp32 sums N_0, D_0, ..., N_3, D_3 (a skipped scale
// 0's two are set to 0 in place).
void scores_from_sums(float sums[8], const vif_options &opt, double out[8]);

// The rows a strip of scale-0 rows [row0, row1) of an h-row frame reads
// (input rows [in0, in0 + in_rows) of the frame) and owns (rows [own0[s],
// own0[s] + nown[s]) of the frame's scale-s plane).  False for a strip the
// boundary does not accept.
struct StripRows {
  int in0, in_rows;
  int own0[kScales], nown[kScales];
};
bool strip_rows(int h, int row0, int row1, StripRows *sr);

// The option checks of the C ABI (vif_options.cpp).
bool options_ok(const vif_options &o);

// Host tap generator (vif_taps.cpp).
int gaussian_taps(int scale, float *taps);

// Geometry of one scale.
struct ScaleGeom {
  int w, h;
  int strips; // ceil(h / kTileH)
  int ntx;    // ceil(w / kTileW)
  size_t tiles() const { return static_cast<size_t>(strips) * ntx; }
};

// Per-scale kernel for n frames (1 <= n <= kMaxBatch): filter, statistic,
// the next scale's planes and the ordered row sums (each row's sum carried
// across the row's tiles inside the kernel).  io.in_* are the scale's planes
// (native samples at scale 0, fp32 planes above); io.next_* receive the next
// scale's planes (unused at scale 3).
hipError_t launch_scale(int scale, int bpc, const ScaleIO &io, int n,
                        const ScaleGeom &g, const TapArgs &taps,
                        const TapArgs &next_taps, const StatArgs &stat,
                        hipStream_t stream);

// Only tile column `col` of scale 0's chained kernel, for one 8-bit frame
// (the check of the hand-over's bounded wait; see vif_selftest.hip).
hipError_t launch_scale0_column(const ScaleIO &io, const ScaleGeom &g,
                                const TapArgs &taps, const TapArgs &next_taps,
                                const StatArgs &stat, int col,
                                hipStream_t stream);

// Scale 0's input staging alone, for n frames of g (io.in_*, io.vec_in,
// io.strips, io.ntx as for launch_scale): every block stages its tile into
// LDS as the scale-0 kernel does and stores the sum of the tile's samples at
// out[tx * n * strips + frame * strips + strip].
hipError_t launch_stage_probe(int bpc, const ScaleIO &io, int n,
                              const ScaleGeom &g, unsigned *out,
                              hipStream_t stream);

// Blocks of the scale-0 kernel the current device keeps resident at once
// (blocks per CU times CUs).
hipError_t scale0_resident_blocks(int bpc, int *blocks);

}  // namespace vifk
