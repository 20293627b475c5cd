// vif_rows.cpp -- host arithmetic on row sums: the sums over rows and the
// scores (shared by every context and by vif_scores_from_rows), and the
// rows a row strip of a frame reads and owns.
#include <cstring>

#include "../../include/vif.h"
#include "vif_internal.h"
#include "vif_status.h"

namespace vifk {

// The host's part of the feature (ADR-1422 "float_vif_sycl computes the
// CPU's arithmetic ...", Decision: the row sums come back from the device
// and the host adds them top to bottom in fp32).  rows holds, scale after
// scale, nrows[s] pairs (n_y, d_y).  N_s and D_s are fp32 sums from 0, rows
// in order; the scores are fp64 quotients; num and den add the four scales
// in order in fp64.  A skipped scale 0 contributes N_0 = D_0 = 0 and reports
// 0.0; the floors act on the reported scores of scales 1..3 only.
// scores_from_sums is the second half: out[8] from the eight sums.
void scores_from_rows(const float *rows, const int nrows[kScales],
                      const vif_options &opt, double out[8], float sums[8]) {
  const float *r = rows;
  for (int s = 0; s < kScales; ++s) {
    float n = 0.0f, d = 0.0f;
    for (int y = 0; y < nrows[s]; ++y) {
      n = n + r[2 * y];
      d = d + r[2 * y + 1];
    }
    r += 2 * nrows[s];
    sums[2 * s] = n;
    sums[2 * s + 1] = d;
  }
  scores_from_sums(sums, opt, out);
}

void scores_from_sums(float sums[8], const vif_options &opt, double out[8]) {
  if (opt.skip_scale0 != 0)
    sums[0] = sums[1] = 0.0f;
  double N[kScales], D[kScales];
  for (int s = 0; s < kScales; ++s) {
    N[s] = static_cast<double>(sums[2 * s]);
    D[s] = static_cast<double>(sums[2 * s + 1]);
    out[s] = N[s] / D[s];
  }
  if (opt.skip_scale0 != 0)
    out[0] = 0.0;
  for (int s = 1; s < kScales; ++s)
    if (out[s] < opt.scale_min_val[s - 1])
      out[s] = opt.scale_min_val[s - 1];
  double num = N[0] + N[1];
  num = num + N[2];
  num = num + N[3];
  double den = D[0] + D[1];
  den = den + D[2];
  den = den + D[3];
  out[4] = num;
  out[5] = den;
  out[6] = num / den;
  out[7] = 0.0;
}

// Rows of a strip: scale-0 rows [row0, row1) of an h-row frame, row0 a
// multiple of 8 and row1 a multiple of 8 or h.  Scale s owns rows
// [row0 >> s, row1 >> s) of its plane (floor(h / 2^s) rows; the last strip
// owns the plane's remaining rows).  To compute them, the kernels need
// scale-0 rows [row0 - 20, row1 + 13) (clamped to the frame): at scale 3 an
// owned row reads the plane's rows one above and below (3 taps); each
// scale-s plane row 2y' is the next scale's low-pass centre, reading 2y' -
// R_{s+1} .. 2y' + R_{s+1} of plane s (radii 4, 2, 1 for scales 1..3); and
// each scale's own terms read radius R_s (8, 4, 2, 1) around them.  Going up
// from scale 3: plane 3 rows [a - 1, b] -> plane 2 [2a - 3, 2b + 1] -> plane
// 1 [4a - 8, 4b + 4] -> plane 0 [8a - 20, 8b + 12], with a = row0 / 8, b =
// row1 / 8; every other need lies inside these.  The first input row is
// rounded down to a multiple of 8 (row0 - 24), so that the strip's planes
// start at a whole row of every scale: plane s of the strip is then rows
// [in0 >> s, ...) of the frame's plane s, its even rows the frame's even
// rows, and the 2x decimation keeps its phase.  Inside the strip the
// kernels mirror at the strip's first and last input rows; those are the
// frame's own edges where the strip reaches them, and elsewhere the rows a
// mirrored index touches feed only halo rows, never an owned one (ADR-1444
// "float_vif_hip runs the arithmetic of the CUDA twin ...", Decision:
// indices reflect at the plane's edge and are then clamped).
bool strip_rows(int h, int row0, int row1, StripRows *sr) {
  if (h < 1 || row0 < 0 || row0 % 8 != 0 || row1 <= row0 || row1 > h ||
      (row1 % 8 != 0 && row1 != h))
    return false;
  const int in0 = row0 >= 24 ? row0 - 24 : 0;
  const int in1 = row1 + 13 <= h ? row1 + 13 : h;
  sr->in0 = in0;
  sr->in_rows = in1 - in0;
  for (int s = 0; s < kScales; ++s) {
    const int first = row0 >> s;
    const int end = row1 == h ? (h >> s) : (row1 >> s);
    sr->own0[s] = first;
    sr->nown[s] = end - first;
  }
  return true;
}

} // namespace vifk

extern "C" {

__attribute__((visibility("default"))) int
vif_strip_geometry(int w, int h, int row0, int row1,
                   int info[VIF_STRIP_INFO]) {
  vifk::StripRows sr;
  if (info == nullptr || w < VIF_MIN_SIDE || h < VIF_MIN_SIDE ||
      static_cast<long>(w) * h > VIF_MAX_PIXELS ||
      !vifk::strip_rows(h, row0, row1, &sr))
    return vifk::set_status(VIF_EINVAL);
  info[0] = sr.in0;
  info[1] = sr.in_rows;
  for (int s = 0; s < vifk::kScales; ++s) {
    info[2 + 2 * s] = sr.own0[s];
    info[3 + 2 * s] = sr.nown[s];
  }
  return vifk::set_status(VIF_OK);
}

__attribute__((visibility("default"))) int
vif_scores_from_rows(int w, int h, const vif_options *opt, const float *rows,
                     double out[8], float sums[8]) {
  vif_options o;
  vif_default_options(&o);
  if (opt != nullptr)
    o = *opt;
  if (rows == nullptr || out == nullptr || w < VIF_MIN_SIDE ||
      h < VIF_MIN_SIDE || static_cast<long>(w) * h > VIF_MAX_PIXELS ||
      !vifk::options_ok(o))
    return vifk::set_status(VIF_EINVAL);
  int nrows[vifk::kScales];
  for (int s = 0; s < vifk::kScales; ++s)
    nrows[s] = h >> s;
  float tmp[8];
  vifk::scores_from_rows(rows, nrows, o, out, sums != nullptr ? sums : tmp);
  return vifk::set_status(VIF_OK);
}

} // extern "C"
