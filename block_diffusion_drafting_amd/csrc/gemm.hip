// Planning and dispatch of the weight-streaming products: grid shape per
// product, and the switch over epilogues (each compiled in its own file).
#include "kernels.h"

namespace dflash {

// ---------------------------------------------------------------------------
// planning and dispatch
// ---------------------------------------------------------------------------
// The grid is sized in whole rounds of 256 workgroups (one per compute
// unit): a workgroup owns a balanced range of up to NTG tiles, and products
// split over k (EPI_PART) use eight splits of about 256 / 8 tile ranges.
// Streaming rate per compute unit is limited by its outstanding misses, so
// a grid that leaves units idle, or gives some two ranges and others one,
// loses bandwidth; measured on the Qwen3-4B-shaped phases on MI355X.
constexpr int kCUs = 256;
// wide_kernel takes the split-K products of five to WIDE_MAX_MTILES m-tiles
// (one to eight 128-row m-groups: K = 80-1024 at batch 1, 256 rows at batch
// 16, verification of up to 1024 rows)
constexpr int WIDE_MAX_MTILES = 64;

// tiles-per-workgroup variants compiled for each m-tile count, and the
// largest one used: with many activation rows a workgroup re-reads every row
// for its tiles, so wider tile ranges cut that traffic (accumulators of up to
// 40 tiles live in the accumulation registers).  Eight m-tiles with the
// hi/lo pair fit four tiles per workgroup without spilling; the k-split
// products (EPI_PART) take five, spilling a few registers, because the
// fewer workgroups re-read less of the activations (measured on the
// Qwen3-4B shape: o + down at K = 128 262 -> 226 us per block, batch 16
// 480 -> 381 us; gate/up and QKV slower with five).  Four m-tiles take at
// most five: with eight a workgroup runs at one wave per SIMD (gate/up in
// 64-row groups at batch 16 516 -> 390 us per block with five); QKV over
// sixteen m-groups or more still gains more from the fewer re-reads (K =
// 1024 630 -> 500 us per block with eight; at eight m-groups, 512 rows,
// eight was slower).
static int max_ntg(int mtt, int epi, int m_groups) {
  if (mtt == 8) return is_part(epi) ? 5 : 4;
  if (mtt == 4) return epi == EPI_QKV && m_groups >= 16 ? 8 : 5;
  return 8;
}
static int round_ntg(int mtt, int cap, int want) {
  static const int v1[] = {1, 2, 4, 5, 6, 8};
  static const int v2[] = {1, 2, 4, 5, 8};
  static const int v4[] = {1, 2, 4, 5, 8};
  static const int v8[] = {1, 2, 4, 5};
  const int* v = mtt == 1 ? v1 : mtt == 2 ? v2 : mtt == 4 ? v4 : v8;
  const int n = mtt == 1 ? 6 : mtt == 8 ? 4 : 5;
  for (int i = 0; i < n && v[i] <= cap; ++i)
    if (v[i] >= want) return v[i];
  return cap;
}

// The context-path products keep a fixed shape at prefill sizes (more than
// two m-tiles: they run once); the per-step ones (the accepted rows, at
// most two m-tiles) use the balanced planning.  EPI_FC (the whole context
// projection in one pass) is only used at prefill sizes.
static bool fixed_shape(int epi, bool rowmajor, int mtt) {
  return epi == EPI_FC || ((epi == EPI_KV || rowmajor) && mtt > 2);
}
static int fixed_ntg(int epi) { return epi == EPI_FC ? 4 : 2; }

GemmPlan plan_gemm(int epi, const Packed& W, int M, bool split_ok, bool rowmajor) {
  GemmPlan p{};
  const int mtiles = (M + 15) / 16;
  p.mtt = mtiles <= 1 ? 1 : mtiles <= 2 ? 2 : mtiles <= 4 ? 4 : 8;
  p.m_groups = (mtiles + p.mtt - 1) / p.mtt;
  p.rowmajor = rowmajor;
  // hi/lo pair for every product but the LM head above two m-tiles: the
  // rounding of its input to bf16 reaches the logits alone, while that of
  // a layer's inputs is carried through the later layers (measured by
  // simulation at the Llama-3.1-8B shape, K = 128: max row error 1.03e-2
  // with the pair everywhere, 1.06e-2 with the LM head's hi part alone,
  // 3.4e-2 with the hi part everywhere)
  p.split = split_ok && !rowmajor && (epi != EPI_ARGMAX || p.mtt <= 2);
  // Smaller m-groups for QKV and gate/up with the hi/lo pair: every
  // workgroup re-reads the whole activation of its m-group from L2, so
  // groups of 32 or 64 rows cut that per workgroup, the weights of a tile
  // range being read once from HBM for all of them (XCD-grouped numbering
  // of gemm_kernel).  Measured at the Qwen3-4B shape: QKV in 32-row groups
  // up to 128 rows (per K = 128 block 185 -> 118 us, K = 64 116 -> 93 us;
  // slower at batch 16, 256 rows) and in 64-row groups above 256 rows
  // (K = 1024 699 -> 500 us), gate/up in 64-row groups unless the head
  // kernel takes it (K = 128 314 -> 240 us, batch 16 600 -> 517 us; 32-row
  // groups slower); the k-split products (o, down) in 32-row groups up to
  // 64 rows (K = 64 214 -> 175 us; slower in 64-row groups at 128 rows).
  if (p.split && ((epi == EPI_QKV && mtiles <= 8) || (is_part(epi) && mtiles <= 4)) && mtiles > 2) {
    p.mtt = 2;
    p.m_groups = (mtiles + 1) / 2;
  } else if (p.split && p.mtt == 8 &&
             ((epi == EPI_QKV && mtiles > 16) ||
              (epi == EPI_SWIGLU && !uses_head_kernel(epi, p, W.n_tiles, 2)))) {
    p.mtt = 4;
    p.m_groups = (mtiles + 3) / 4;
  }
  const int T = W.n_tiles;
  // One to eight 128-row m-groups with the hi/lo pair: the split-K product
  // (EPI_PART, the output and down projections above four m-tiles) runs
  // wide_kernel, eight tiles per workgroup (four per wave slot), with about
  // one round of workgroups over its tile groups and m-groups and splits of
  // at least eight k-blocks.  Measured at the Qwen3-4B shape, per launch: o
  // + down average 21.1 -> 16.2 us at 128 rows (down 29 -> about 22 us with
  // 12 splits), 36.7 -> 23.5 us at 256 rows (batch 16); per block at 1024
  // rows o 0.44 -> 0.30 ms and down 0.94 -> 0.66 ms.  Gate/up on wide_kernel
  // was no faster than gemm_kernel in 64-row groups (46.2 vs 46.3 us at 128
  // rows), so it stays there.
  if (p.split && mtiles > 4 && mtiles <= WIDE_MAX_MTILES && epi == EPI_PART && !rowmajor) {
    p.wide = true;
    p.mtt = 8;
    p.m_groups = (mtiles + 7) / 8;
    p.ntg = 4;
    p.n_groups = (T + 2 * p.ntg - 1) / (2 * p.ntg);
    int ns = kCUs / (p.n_groups * p.m_groups);
    if (ns > W.nkb / 8) ns = W.nkb / 8;
    if (ns < 1) ns = 1;
    p.kbu = (W.nkb + ns - 1) / ns;
    p.nsplit = (W.nkb + p.kbu - 1) / p.kbu;
    p.part_floats = (size_t)p.nsplit * T * mtiles * 256;
    p.fixed = false;
    return p;
  }
  if (is_part(epi)) {
    int ns = MAX_SPLITS;
    while (ns > 1 && W.nkb / ns < 8) ns /= 2;
    p.kbu = (W.nkb + ns - 1) / ns;
    p.nsplit = (W.nkb + p.kbu - 1) / p.kbu;
    p.part_floats = (size_t)p.nsplit * T * mtiles * 256;
  } else {
    p.kbu = W.nkb;
    p.nsplit = 1;
    p.part_floats = 0;
  }
  p.fixed = fixed_shape(epi, rowmajor, p.mtt);
  if (p.fixed) {
    p.ntg = fixed_ntg(epi);
    p.n_groups = (T + p.ntg - 1) / p.ntg;
    return p;
  }
  const int per_round = kCUs / (p.nsplit * p.m_groups) > 0 ? kCUs / (p.nsplit * p.m_groups) : 1;
  const int cap = max_ntg(p.mtt, epi, p.m_groups);
  int groups = per_round * ((T + per_round * cap - 1) / (per_round * cap));
  if (groups > T) groups = T;
  p.ntg = round_ntg(p.mtt, cap, (T + groups - 1) / groups);
  p.n_groups = groups;
  return p;
}

template <typename T>
hipError_t launch_gemm(int epi, const GemmPlan& p, const GemmArgs& g, const EpiArgs& e,
                       hipStream_t s) {
  switch (epi) {
    case EPI_QKV: return launch_gemm_epi<T, EPI_QKV>(p, g, e, s);
    case EPI_SWIGLU: return launch_gemm_epi<T, EPI_SWIGLU>(p, g, e, s);
    case EPI_PART: return launch_gemm_epi<T, EPI_PART>(p, g, e, s);
    case EPI_ARGMAX: return launch_gemm_epi<T, EPI_ARGMAX>(p, g, e, s);
    case EPI_FC: return launch_gemm_epi<T, EPI_FC>(p, g, e, s);
    case EPI_KV: return launch_gemm_epi<T, EPI_KV>(p, g, e, s);
    case EPI_RESNORM: return launch_gemm_epi<T, EPI_RESNORM>(p, g, e, s);
    case EPI_PARTRES: return launch_gemm_epi<T, EPI_PARTRES>(p, g, e, s);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_gemm<bf16_t>(int, const GemmPlan&, const GemmArgs&, const EpiArgs&, hipStream_t);
template hipError_t launch_gemm<float>(int, const GemmPlan&, const GemmArgs&, const EpiArgs&, hipStream_t);


}  // namespace dflash
