// C ABI of the EQ-Linear library (declared in include/eqlinear.h): argument
// validation, tile / split policy and launches on the caller's stream.  Nothing
// here allocates device memory or synchronises the host.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "eql_launch.h"
#include "eqlinear.h"

using namespace eql;

namespace {

constexpr int64_t kMaxGrid = (1LL << 24) - 1;  // workgroups per launch (x 256 threads < 2^32)
constexpr int kTargetWorkgroups = 256;         // one per compute unit of an MI355X
constexpr int64_t kMaxRowBytes = 1LL << 23;    // bytes of one activation row (buffer offsets)

bool dtype_ok(int dtype) { return dtype == EQL_F32 || dtype == EQL_F16; }
int elt_bytes(int dtype) { return dtype == EQL_F16 ? 2 : 4; }
int group_channels(int dtype) { return 16 / elt_bytes(dtype); }
// 16-byte channel groups of the packed weight's input axis, padded to a whole
// number of kernel K stages (kPackGroupAlign groups).
int64_t padded_groups(int64_t ch, int dtype) {
  const int64_t g = (ch + group_channels(dtype) - 1) / group_channels(dtype);
  return (g + kPackGroupAlign - 1) / kPackGroupAlign * kPackGroupAlign;
}
// Output channels of the packed weight, padded to whole 32-channel blocks.
int64_t padded_out(int64_t ch) { return (ch + kPackBlock - 1) / kPackBlock * kPackBlock; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// cos / sin(2 pi m / T), m = 0..T-1: computed in double with the C library and
// rounded once to float.
Twiddles make_twiddles(int T) {
  Twiddles tw{};
  const double two_pi = 6.28318530717958647692528676655900577;
  for (int m = 0; m < T; ++m) {
    tw.cs[m] = (float)std::cos(two_pi * m / T);
    tw.sn[m] = (float)std::sin(two_pi * m / T);
  }
  tw.inv_t = (float)(1.0 / T);
  return tw;
}

// Rows: a row index plus any kernel's row-block size (at most 1024) stays below 2^31.
constexpr int64_t kMaxN = (1LL << 31) - (1LL << 20);

int check_sizes(int64_t N, int64_t Cp, int64_t Dp, int T, int dtype) {
  if (!dtype_ok(dtype) || T < 1) return EQL_EINVAL;
  if (T > EQL_MAX_T) return EQL_EUNSUPPORTED;
  if (N < 0 || Cp < 1 || Dp < 1) return EQL_EINVAL;
  // Row widths compared by division first: Cp or Dp near INT64_MAX must not overflow.
  const int64_t maxCh = kMaxRowBytes / (T * elt_bytes(dtype));
  if (N > kMaxN || Cp > maxCh || Dp > maxCh) return EQL_EINVAL;
  return EQL_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? EQL_OK : EQL_EHIP; }

// Fixed per-stage cost of a forward tile in units of one 32-column block's MFMAs.
constexpr int64_t kFwdStageFixed = 5;
// A tile's epilogue (inverse transform and stores, not overlapped with MFMAs) per
// 32-column block, in the same units.
constexpr int64_t kFwdEpilogueBlock = 21;

// Compute units of the current device (cached per device; 256 on MI355X).  The
// persistent kernels launch one workgroup per compute unit.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kTargetWorkgroups;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = kTargetWorkgroups;
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Shared by the forward pass and the input gradient: out = in * W^T for the packed
// weight with (out, in) channel counts (Dout, Cin).
// epi: the fused epilogue (bias, act, res); otherwise those are ignored.
// Relative cost of a forward tile that also stores its transformed input (the stores
// and the transposes), in percent of a plain tile's; EQL_SPEC_COST overrides it (for
// measurement).
int spec_cost_pct() {
  static const int v = [] {
    const char* e = std::getenv("EQL_SPEC_COST");
    const int p = e ? std::atoi(e) : 0;
    return p >= 50 && p <= 400 ? p : 175;
  }();
  return v;
}

// Workgroups of the spectrum-storing forward launch that take column 0's row tiles: a
// multiple of 8 (one per XCD each), so that both parts keep the XCD-aware tile order,
// chosen to balance rounds of column-0 tiles (weighted by spec_cost_pct) against rounds
// of the other columns on the remaining compute units.
int spec_grid(int64_t rowTiles, int64_t colTiles, int cus) {
  const int64_t plain = rowTiles * (colTiles - 1);
  const int maxGs = std::max(8, cus / 8 * 8);
  if (plain == 0) return (int)std::min<int64_t>(ceil_div(rowTiles, 8) * 8, maxGs);
  int best = 8;
  int64_t bestCost = -1;
  for (int gs = 8; gs < maxGs; gs += 8) {
    const int gp = cus - gs;
    const int64_t cost = std::max(ceil_div(rowTiles, gs) * spec_cost_pct(), ceil_div(plain, gp) * 100);
    if (bestCost < 0 || cost < bestCost) {
      bestCost = cost;
      best = gs;
    }
  }
  return best;
}

// spec: also store the transformed input as weight-gradient operand units into this
// section of specBytes bytes, channel axis padded to specKpad (fwd_spec_ok must hold).
int run_fwd(const void* x, const void* wp, void* y, int64_t N, int64_t Cin, int64_t Dout, int T,
            int dtype, void* stream, bool epi = false, const void* bias = nullptr, const void* res = nullptr,
            int act = 0, void* pre = nullptr, void* spec = nullptr, int64_t specKpad = 0, size_t specBytes = 0) {
  int st = check_sizes(N, Cin, Dout, T, dtype);
  if (st != EQL_OK) return st;
  if (N == 0) return EQL_OK;
  if (!x || !wp || !y) return EQL_EINVAL;
  if (!aligned16(x) || !aligned16(wp) || !aligned16(y)) return EQL_EALIGN;

  const int nbm = fwd_nb_max(T);
  const int64_t rowTiles = ceil_div(N, kFwdRows);
  const bool rowsAligned = (Cin * T * elt_bytes(dtype)) % 16 == 0;
  const int cus = device_cus();
  // Tile width (32-column blocks): the persistent grid takes ceil(tiles / CUs) rounds,
  // and a tile costs about kFwdStageFixed + nb block-units per K stage (the stage's
  // barrier, x load and transform measure about five blocks' MFMA time) plus
  // kFwdEpilogueBlock per block for its epilogue, which weighs in on short K (c2's
  // forward, 6 stages: 64-column tiles 8% faster than 128-column ones, as this predicts).
  // Fewest estimated units wins; ties go to the wider tile, which moves fewer bytes per
  // FLOP.  EQL_FWD_NB=1|2|4 forces the width where it applies (for measurement).
  int nb = 1;
  if (rowsAligned) {
    int64_t best = -1;
    static const int forcedNb = [] {
      const char* v = std::getenv("EQL_FWD_NB");
      return v && (std::strcmp(v, "1") == 0 || std::strcmp(v, "2") == 0 || std::strcmp(v, "4") == 0) ? std::atoi(v) : 0;
    }();
    for (int cand = nbm; cand >= 1; cand /= 2) {
      if (forcedNb && cand != forcedNb && forcedNb <= nbm) continue;
      const int64_t rounds = ceil_div(rowTiles * ceil_div(Dout, 32 * cand), (int64_t)cus);
      const int64_t nst = padded_groups(Cin, dtype) / 2;
      const int64_t cost = rounds * (nst * (kFwdStageFixed + cand) + kFwdEpilogueBlock * cand);
      if (best < 0 || cost < best) {
        best = cost;
        nb = cand;
      }
    }
  }
  const int64_t colTiles = ceil_div(Dout, 32 * nb);
  if (colTiles > kMaxGrid) return EQL_EINVAL;

  FwdArgs a{};
  a.wp = wp;
  a.Cin = (int)Cin;
  a.Dout = (int)Dout;
  a.Jpad = (int)padded_groups(Cin, dtype);
  const int64_t wpBytes = padded_out(Dout) * a.Jpad * 16LL * T;
  if (wpBytes >= (1LL << 32)) return EQL_EINVAL;
  a.wpBytes = (uint32_t)wpBytes;
  a.colTiles = (int)colTiles;
  a.loadMode = !rowsAligned ? kLoadNarrow
               : (Cin % ((int64_t)kPackGroupAlign * group_channels(dtype)) == 0 ? kLoadFull : kLoadAligned);
  a.tw = make_twiddles(T);
  a.bias = bias;
  a.act = act;

  // Rows in pieces small enough for the tile indices.
  const int64_t maxRows = (kMaxGrid / colTiles) * kFwdRows;
  const size_t inRow = (size_t)Cin * T * elt_bytes(dtype), outRow = (size_t)Dout * T * elt_bytes(dtype);
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t r0 = 0; r0 < N; r0 += maxRows) {
    const int64_t rows = N - r0 < maxRows ? N - r0 : maxRows;
    a.x = static_cast<const char*>(x) + (size_t)r0 * inRow;
    a.y = static_cast<char*>(y) + (size_t)r0 * outRow;
    a.res = res ? static_cast<const char*>(res) + (size_t)r0 * outRow : nullptr;
    a.pre = pre ? static_cast<char*>(pre) + (size_t)r0 * outRow : nullptr;
    if (spec) {
      // r0 is a multiple of the row tile, so of the 16 rows of one k-step.
      const size_t skip = (size_t)(r0 / 16) * (size_t)T * 2 * (size_t)specKpad * 16;
      a.spec = static_cast<char*>(spec) + skip;
      a.specBytes = (uint32_t)(specBytes - skip);
      a.specKpad = (int)specKpad;
    }
    a.N = (int)rows;
    const int64_t rowTiles = ceil_div(rows, kFwdRows);
    a.numTiles = (int)(rowTiles * colTiles);
    hipError_t e;
    if (spec) {
      const int gs = spec_grid(rowTiles, colTiles, cus);
      a.specGrid = gs;
      const int64_t plain = rowTiles * (colTiles - 1);
      const unsigned grid = (unsigned)(gs + std::min<int64_t>(plain, std::max(cus - gs, 8)));
      e = launch_fwd_spec_f16(nb, epi, a, grid, s);
    } else {
      const unsigned grid = (unsigned)std::min<int64_t>(a.numTiles, cus);
      e = epi ? (dtype == EQL_F16 ? launch_fwd_fused_f16(T, nb, a, grid, s) : launch_fwd_fused_f32(T, nb, a, grid, s))
              : (dtype == EQL_F16 ? launch_fwd_f16(T, nb, a, grid, s) : launch_fwd_f32(T, nb, a, grid, s));
    }
    if (e != hipSuccess) return EQL_EHIP;
  }
  return EQL_OK;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Weight-gradient plan.  The workspace holds, in order (each section 256-byte
// aligned): the half spectra of dy and of x as MFMA operand units (2G rows per
// k-step, zero rows past N, channels padded to a multiple of the GEMM tile width),
// then the fp32 partial spectra of the real-plane GEMM [SR][NR][Dp][Cp] and of the
// complex-pair GEMM [SP][T-NR][Dp][Cp].
struct GemmPlan {
  int DB = 1, CB = 1, WCN = 2;  // 2 x WCN waves of DB x CB blocks: tile 64 DB x 32 CB WCN
  int64_t groups = 0, dTiles = 0, cTiles = 0, S = 0, kgPerSplit = 0;
  int64_t items() const { return S * groups * dTiles * cTiles; }
};

// Tile width of one channel axis: 256 unless padding to it adds more than a third
// of the channels, else 64.
int64_t tile_width(int64_t ch) { return ceil_div(ch, 256) * 256 * 3 <= ch * 4 ? 256 : 64; }

struct BwdwPlan {
  int64_t kgCount = 0, Dpad = 0, Cpad = 0;
  GemmPlan real, pair;
  // Fused path (dy transformed inside the GEMM, eql_bwdw4_kernel): one launch over
  // S x dTiles x cTiles items of 128 x 128 output channels, all planes.
  bool fused = false;
  int fNB = 4;  // 32-channel blocks of c per tile
  int64_t fS = 0, fKgPerSplit = 0, fDTiles = 0, fCTiles = 0;
  size_t dyhBytes = 0, xhBytes = 0, partRBytes = 0, partPBytes = 0;
  size_t total() const { return dyhBytes + xhBytes + partRBytes + partPBytes; }
};

// Which weight-gradient path a shape takes.  The fused path (dy's transform inside
// the GEMM, all T planes per tile) reads dy once and never writes its spectrum, but
// its 128 x 128 x T tiles move more operand bytes per MFMA than the separate path's
// per-plane tiles.  It wins where the layer is bound by memory traffic: actual FLOPs
// per algorithmic byte below kFusedIntensity (the fp16 MFMA / HBM ridge is about
// 315).  It needs T in {1, 2, 4} and 16-byte dy rows.  The environment variable
// EQL_BWDW_PATH=fused|separate overrides the choice where the fused path applies
// (for measurement).
constexpr double kFusedIntensity = 400.0;

bool bwdw_fused(int64_t N, int64_t Cp, int64_t Dp, int T, int dtype) {
  const int elt = elt_bytes(dtype);
  if (N == 0 || !(T == 1 || T == 2 || T == 4) || (Dp * T * elt) % 16 != 0) return false;
  if ((double)N * (double)(Dp * T * elt) >= 4294967296.0) return false;  // dy within one 32-bit range
  static const int forced = [] {
    const char* v = std::getenv("EQL_BWDW_PATH");
    if (v && std::strcmp(v, "fused") == 0) return 1;
    if (v && std::strcmp(v, "separate") == 0) return 2;
    return 0;
  }();
  if (forced) return forced == 1;
  const double planes = T == 1 ? 1.0 : (T == 2 ? 2.0 : 6.0);  // real products per (d, c) pair
  const double flops = 2.0 * planes * (double)N * (double)Dp * (double)Cp;
  const double bytes = (double)elt * T * (double)N * (double)(Cp + Dp);
  return flops / bytes < kFusedIntensity;
}

// Waves per workgroup of the separate path's GEMMs on 256-wide tiles, for the real-plane
// GEMM (pair = false) and the complex-pair GEMM.  EQL_BWDW_WAVES=4|8 overrides both,
// EQL_BWDW_WAVES=<real>,<pair> (e.g. 4,8) each (for measurement).
int bwdw_waves(bool pair) {
  static const int forced = [] {
    const char* v = std::getenv("EQL_BWDW_WAVES");
    if (!v) return 0;
    if (std::strcmp(v, "4") == 0) return 44;
    if (std::strcmp(v, "8") == 0) return 88;
    if (std::strcmp(v, "4,8") == 0) return 48;
    if (std::strcmp(v, "8,4") == 0) return 84;
    return 0;
  }();
  if (!forced) return 8;
  return pair ? forced % 10 : forced / 10;
}

constexpr int64_t kMinStepsPerSplit = 16;  // keeps partial-spectrum traffic small
// Small layers may split down to kMinStepsSmall k-steps per row range while their
// partials stay within kSmallPartialBytes: few outputs and few rows would otherwise
// leave a handful of workgroups each walking a long serial chain of stages.
constexpr int64_t kMinStepsSmall = 2;
constexpr int64_t kSmallPartialBytes = 1 << 20;

// Row ranges of a reduction over kgCount k-steps for `tiles` output items whose
// partials take partBytesPerSplit bytes per range: enough ranges to give every compute
// unit one item.
int64_t split_count(int64_t tiles, int64_t kgCount, int64_t partBytesPerSplit) {
  const int64_t want = tiles >= kTargetWorkgroups ? 1 : kTargetWorkgroups / tiles;
  int64_t S = std::min<int64_t>(want, std::max<int64_t>(1, kgCount / kMinStepsPerSplit));
  if (S < want) {
    const int64_t S2 = std::min<int64_t>(want, std::max<int64_t>(1, kgCount / kMinStepsSmall));
    if (S2 * partBytesPerSplit <= kSmallPartialBytes) S = S2;
  }
  return S;
}

// Row ranges (k-step ranges) of one GEMM launch.
void plan_splits(GemmPlan& g, int64_t kgCount, int64_t partBytesPerSplit) {
  const int64_t tiles = g.groups * g.dTiles * g.cTiles;
  if (tiles == 0 || kgCount == 0) return;
  const int64_t S = split_count(tiles, kgCount, partBytesPerSplit);
  g.kgPerSplit = ceil_div(kgCount, S);
  g.S = ceil_div(kgCount, g.kgPerSplit);
}

BwdwPlan plan_bwdw(int64_t N, int64_t Cp, int64_t Dp, int T, int dtype) {
  BwdwPlan p;
  const int nr = n_real_planes(T), np = n_pairs(T);
  const int64_t wd = tile_width(Dp), wc = tile_width(Cp);
  p.Dpad = ceil_div(Dp, wd) * wd;
  p.Cpad = ceil_div(Cp, wc) * wc;
  // Real planes: wd x wc tiles; complex pairs hold two planes, so half as wide in c
  // (at least 64).
  p.real.DB = (int)(wd / 64);
  p.real.CB = (int)(wc / 64);
  p.pair.DB = p.real.DB;
  p.pair.CB = wc == 256 ? 2 : 1;
  // 256 x 256 (real) and 256 x 128 (pair) tiles: 8 waves, two per SIMD, each with half
  // the columns of the 4-wave arrangement.
  if (wd == 256 && wc == 256) {
    if (bwdw_waves(false) == 8) {
      p.real.CB = 2;
      p.real.WCN = 4;
    }
    if (bwdw_waves(true) == 8) {
      p.pair.CB = 1;
      p.pair.WCN = 4;
    }
  }
  p.real.groups = nr;
  p.real.dTiles = p.Dpad / wd;
  p.real.cTiles = p.Cpad / wc;
  p.pair.groups = np;
  p.pair.dTiles = p.Dpad / wd;
  p.pair.cTiles = p.Cpad / (32 * p.pair.CB * p.pair.WCN);
  if (N == 0) return p;
  p.kgCount = ceil_div(N, 2 * group_channels(dtype));
  if (bwdw_fused(N, Cp, Dp, T, dtype)) {
    p.fused = true;
    // Column tile of 32 NB channels: the least padding of C', ties to the wider tile;
    // the tile's spectrum stage (T NB KB) must split evenly over the four waves.
    int64_t best = -1;
    for (int nb = 4; nb >= 2; --nb) {
      if ((T * nb) % 4 != 0) continue;
      const int64_t padded = ceil_div(Cp, 32 * nb) * 32 * nb;
      if (best < 0 || padded < best) {
        best = padded;
        p.fNB = nb;
      }
    }
    p.fDTiles = ceil_div(Dp, kBwdw4Tile);
    p.fCTiles = ceil_div(Cp, 32 * p.fNB);
    p.Cpad = p.fCTiles * 32 * p.fNB;
    const int64_t tiles = p.fDTiles * p.fCTiles;
    const int64_t S = split_count(tiles, p.kgCount, (int64_t)T * Dp * Cp * (int64_t)sizeof(float));
    p.fKgPerSplit = ceil_div(p.kgCount, S);
    p.fS = ceil_div(p.kgCount, p.fKgPerSplit);
    p.real.S = p.pair.S = p.fS;
    p.xhBytes = align256((size_t)p.kgCount * T * 2 * (size_t)p.Cpad * 16);
    p.partRBytes = align256((size_t)p.fS * nr * (size_t)Dp * (size_t)Cp * sizeof(float));
    p.partPBytes = (size_t)p.fS * (T - nr) * (size_t)Dp * (size_t)Cp * sizeof(float);
    return p;
  }
  plan_splits(p.real, p.kgCount, (int64_t)nr * Dp * Cp * (int64_t)sizeof(float));
  plan_splits(p.pair, p.kgCount, (int64_t)(T - nr) * Dp * Cp * (int64_t)sizeof(float));
  p.dyhBytes = align256((size_t)p.kgCount * T * 2 * (size_t)p.Dpad * 16);
  p.xhBytes = align256((size_t)p.kgCount * T * 2 * (size_t)p.Cpad * 16);
  p.partRBytes = align256((size_t)p.real.S * nr * (size_t)Dp * (size_t)Cp * sizeof(float));
  p.partPBytes = (size_t)p.pair.S * (T - nr) * (size_t)Dp * (size_t)Cp * sizeof(float);
  return p;
}

// Whether the forward kernel itself can store the transformed input (Cin channels)
// as weight-gradient operand units into a section of `bytes` bytes with the channel
// axis padded to Kpad: p4 fp16 with 16-byte rows (the ring kernel), and the section
// plus the last row tile's overhang (at most 8 k-steps past it) within 31-bit
// offsets.
bool fwd_spec_ok(int64_t Cin, int T, int dtype, size_t bytes, int64_t Kpad) {
  if (T != 4 || dtype != EQL_F16 || (Cin * T * elt_bytes(dtype)) % 16 != 0) return false;
  return (double)bytes + 8.0 * T * 2 * (double)Kpad * 16 < 2147483648.0;
}

// The group transform of one N x K matrix (x or dy) into operand units [kg][T][2][Kpad]
// by eql_spec_kernel.
int run_spec(const void* m, void* out, int64_t N, int64_t K, int64_t Kpad, int64_t kgCount, int T, int dtype,
             hipStream_t s) {
  const int64_t grid = ceil_div(kgCount * 2 * Kpad, 256);
  if (grid > kMaxGrid) return EQL_EINVAL;
  SpecArgs sp{};
  sp.N = (int)N;
  sp.kgCount = (int)kgCount;
  sp.tw = make_twiddles(T);
  sp.m = m;
  sp.out = out;
  sp.K = (int)K;
  sp.Kpad = (int)Kpad;
  sp.blocks1 = (int)grid;
  return status_of(dtype == EQL_F16 ? launch_spec_f16(T, sp, (unsigned)grid, s)
                                    : launch_spec_f32(T, sp, (unsigned)grid, s));
}

// Launch shape of the epilogue backward: chunk width W (the widest power of two, up
// to 16 bytes, dividing a row), 64 chunks across per workgroup, and rows per
// workgroup halved from 1024 (down to 16) until the grid has 2048 workgroups (eight
// per compute unit) or more.  The bias partials take one fp32 per row block and
// element position.
struct EpiPlan {
  int W;
  int64_t rowsPerBlock, rowBlocks, chunkBlocks;
  size_t partBytes;
};

EpiPlan plan_epi(int64_t N, int64_t Dp, int T, int dtype) {
  EpiPlan p{};
  const int64_t rowBytes = Dp * T * elt_bytes(dtype);
  p.W = pow2_part((int)(rowBytes % 16 == 0 ? 16 : rowBytes % 16));
  p.chunkBlocks = ceil_div(rowBytes / p.W, 64);
  p.rowsPerBlock = 1024;
  while (p.rowsPerBlock > 16 && ceil_div(N, p.rowsPerBlock) * p.chunkBlocks < 2048) p.rowsPerBlock /= 2;
  p.rowBlocks = ceil_div(N, p.rowsPerBlock);
  p.partBytes = (size_t)p.rowBlocks * (size_t)(Dp * T) * sizeof(float);
  return p;
}

// Scratch of eqlinear_fused_epilogue_bwd_noalloc: the bias gradient's row-block
// column sums of one call.  Each device holds its own copy, at its own address,
// until the process ends; host code uses the address hipGetSymbolAddress returns on
// that device, never the array's name (a host-side stand-in).
constexpr size_t kScratchBytes = EQL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch[kMaxDevices];

// `scratch` on the current device, looked up once per device with that device
// current; null if the device or the lookup fails.
float* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* addr = nullptr;
  if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
  // Every thread that races here gets the same address; any of them may store it.
  g_scratch[dev].store(static_cast<float*>(addr), std::memory_order_release);
  return static_cast<float*>(addr);
}

// Body of both epilogue-backward entry points.  noalloc: the partials go to the
// current device's `scratch` instead of the caller's workspace (workspace and
// ws_bytes are ignored).
int epilogue_bwd(const void* dy, const void* pre, void* dpre, void* dbias, void* workspace, size_t ws_bytes,
                 int64_t N, int64_t Dp, int T, int dtype, int act, void* stream, bool noalloc) {
  if (act != EQL_ACT_NONE && act != EQL_ACT_GELU) return EQL_EINVAL;
  int st = check_sizes(N, 1, Dp, T, dtype);
  if (st != EQL_OK) return st;
  const EpiPlan p = plan_epi(N, Dp, T, dtype);
  if (p.rowBlocks * p.chunkBlocks > kMaxGrid) return EQL_EINVAL;
  if (N > 0 && (!dy || !dpre || (act == EQL_ACT_GELU && !pre))) return EQL_EINVAL;
  const bool parts = dbias && N > 0;
  if (noalloc) {
    if (parts && p.partBytes > kScratchBytes) return EQL_ESCRATCH;
  } else if (parts && (!workspace || ws_bytes < p.partBytes)) {
    return EQL_EINVAL;
  }
  if ((dy && !aligned16(dy)) || (pre && !aligned16(pre)) || (dpre && !aligned16(dpre)) ||
      (workspace && !aligned16(workspace)) ||
      (dbias && (reinterpret_cast<uintptr_t>(dbias) % (uintptr_t)elt_bytes(dtype)) != 0))
    return EQL_EALIGN;
  if (noalloc && parts) {
    workspace = scratch_on_current_device();
    if (!workspace) return EQL_EHIP;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f16 = dtype == EQL_F16;
  EpiBwdArgs a{};
  a.dy = dy;
  a.pre = pre;
  a.dpre = dpre;
  a.part = parts ? static_cast<float*>(workspace) : nullptr;
  a.dbias = dbias;
  a.N = (int)N;
  a.Dp = (int)Dp;
  a.T = T;
  a.act = act;
  a.rowElems = (int)(Dp * T);
  a.rowsPerBlock = (int)p.rowsPerBlock;
  a.chunkBlocks = (int)p.chunkBlocks;
  a.rowBlocks = N > 0 ? (int)p.rowBlocks : 0;
  if (N > 0) {
    const hipError_t e = launch_epi_bwd(f16, p.W, a, (unsigned)(p.rowBlocks * p.chunkBlocks), s);
    if (e != hipSuccess) return EQL_EHIP;
  }
  // dbias (zeros when N == 0: no partials to add).
  if (dbias) return status_of(launch_epi_bias(f16, a, (unsigned)ceil_div(Dp, 16), s));
  return EQL_OK;
}

// Body of the weight-gradient entry points.  spectra: the workspace already holds x's
// spectrum and, on the separate path, dy's (written by the training forward and
// input gradient); only the GEMMs and the reduce run, and x is not read.
int run_bwdw(const void* x, const void* dy, void* dw, void* workspace, size_t ws_bytes, int64_t N, int64_t Cp,
             int64_t Dp, int T, int dtype, void* stream, bool spectra) {
  int st = check_sizes(N, Cp, Dp, T, dtype);
  if (st != EQL_OK) return st;
  const BwdwPlan p = plan_bwdw(N, Cp, Dp, T, dtype);
  const bool needX = !spectra, needDy = !spectra || p.fused;
  if (!dw || (N > 0 && ((needX && !x) || (needDy && !dy) || !workspace))) return EQL_EINVAL;
  if (ws_bytes < p.total()) return EQL_EINVAL;
  if (!aligned16(dw) || (N > 0 && ((needX && !aligned16(x)) || (needDy && !aligned16(dy)) || !aligned16(workspace))))
    return EQL_EALIGN;
  const int64_t gdy = ceil_div(p.kgCount * 2 * p.Dpad, 256);
  const int64_t gx = ceil_div(p.kgCount * 2 * p.Cpad, 256);
  const int rwaves = reduce_waves(p.real.S * n_real_planes(T) + p.pair.S * (T - n_real_planes(T)), Dp * Cp);
  const int64_t rgrid = ceil_div(Dp * Cp, 256 / rwaves);
  const int64_t fItems = p.fS * p.fDTiles * p.fCTiles;
  if (p.real.items() > kMaxGrid || p.pair.items() > kMaxGrid || gdy + gx > kMaxGrid ||
      rgrid > kMaxGrid || fItems > kMaxGrid)
    return EQL_EINVAL;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const Twiddles tw = make_twiddles(T);
  char* ws = static_cast<char*>(workspace);
  float* partR = reinterpret_cast<float*>(ws + p.dyhBytes + p.xhBytes);
  float* partP = reinterpret_cast<float*>(ws + p.dyhBytes + p.xhBytes + p.partRBytes);
  const bool f16 = dtype == EQL_F16;
  if (N > 0 && p.fused) {
    // x's spectrum only; dy is transformed inside the GEMM.
    if (!spectra) {
      st = run_spec(x, ws, N, Cp, p.Cpad, p.kgCount, T, dtype, s);
      if (st != EQL_OK) return st;
    }
    Bwdw4Args a{};
    a.dy = dy;
    a.xh = ws;
    a.wsR = partR;
    a.wsP = partP;
    a.N = (int)N;
    a.Dp = (int)Dp;
    a.Cp = (int)Cp;
    a.Cpad = (int)p.Cpad;
    a.kgCount = (int)p.kgCount;
    a.kgPerSplit = (int)p.fKgPerSplit;
    a.dTiles = (int)p.fDTiles;
    a.cTiles = (int)p.fCTiles;
    a.numItems = (int)fItems;
    a.tw = tw;
    if (launch_bwdw4(f16, T, p.fNB, a, (unsigned)fItems, s) != hipSuccess) return EQL_EHIP;
  } else if (N > 0) {
    hipError_t e = hipSuccess;
    if (!spectra) {
      // dy's and x's spectra in one launch: dy's workgroups first, then x's.
      SpecArgs sp{};
      sp.N = (int)N;
      sp.kgCount = (int)p.kgCount;
      sp.tw = tw;
      sp.m = dy;
      sp.out = ws;
      sp.K = (int)Dp;
      sp.Kpad = (int)p.Dpad;
      sp.m2 = x;
      sp.out2 = ws + p.dyhBytes;
      sp.K2 = (int)Cp;
      sp.Kpad2 = (int)p.Cpad;
      sp.blocks1 = (int)gdy;
      e = f16 ? launch_spec_f16(T, sp, (unsigned)(gdy + gx), s) : launch_spec_f32(T, sp, (unsigned)(gdy + gx), s);
      if (e != hipSuccess) return EQL_EHIP;
    }
    for (int pair = 0; pair < 2; ++pair) {
      const GemmPlan& g = pair ? p.pair : p.real;
      if (g.items() == 0) continue;
      BwdwArgs a{};
      a.dyh = ws;
      a.xh = ws + p.dyhBytes;
      a.ws = pair ? partP : partR;
      a.Dp = (int)Dp;
      a.Cp = (int)Cp;
      a.Dpad = (int)p.Dpad;
      a.Cpad = (int)p.Cpad;
      a.kgCount = (int)p.kgCount;
      a.kgPerSplit = (int)g.kgPerSplit;
      a.groups = (int)g.groups;
      a.dTiles = (int)g.dTiles;
      a.cTiles = (int)g.cTiles;
      a.numItems = (int)g.items();
      if (pair)
        e = f16 ? launch_bwdw_pair_f16(T, g.DB, g.CB, g.WCN, a, (unsigned)a.numItems, s)
                : launch_bwdw_pair_f32(T, g.DB, g.CB, g.WCN, a, (unsigned)a.numItems, s);
      else
        e = f16 ? launch_bwdw_real_f16(T, g.DB, g.CB, g.WCN, a, (unsigned)a.numItems, s)
                : launch_bwdw_real_f32(T, g.DB, g.CB, g.WCN, a, (unsigned)a.numItems, s);
      if (e != hipSuccess) return EQL_EHIP;
    }
  }
  BwdwReduceArgs r{};
  r.wsR = partR;
  r.wsP = partP;
  r.dw = dw;
  r.SR = (int)p.real.S;
  r.SP = (int)p.pair.S;
  r.Dp = (int)Dp;
  r.Cp = (int)Cp;
  r.tw = tw;
  return status_of(f16 ? launch_bwdw_reduce_f16(T, rwaves, r, (unsigned)rgrid, s)
                       : launch_bwdw_reduce_f32(T, rwaves, r, (unsigned)rgrid, s));
}

}  // namespace

extern "C" {

int eqlinear_abi_version(void) { return 205; }

const char* eqlinear_status_string(int status) {
  switch (status) {
    case EQL_OK: return "ok";
    case EQL_EINVAL: return "invalid argument (null pointer, size out of range, unknown dtype or mode, or workspace too small)";
    case EQL_EALIGN: return "a base pointer is not 16-byte aligned";
    case EQL_EUNSUPPORTED: return "group order T above EQL_MAX_T";
    case EQL_EHIP: return "HIP launch failed";
    case EQL_ESCRATCH: return "the shape needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

size_t eqlinear_packed_weight_bytes(int64_t out_ch, int64_t in_ch, int T, int dtype) {
  if (check_sizes(0, in_ch, out_ch, T, dtype) != EQL_OK) return 0;
  return (size_t)padded_out(out_ch) * (size_t)padded_groups(in_ch, dtype) * 16 * T;
}

int eqlinear_pack_weight(const void* w, void* w_packed, int64_t Dp, int64_t Cp, int T, int dtype,
                         int mode, void* stream) {
  int st = check_sizes(0, Cp, Dp, T, dtype);
  if (st != EQL_OK) return st;
  if (mode != EQL_PACK_FWD && mode != EQL_PACK_BWDX) return EQL_EINVAL;
  if (!w || !w_packed) return EQL_EINVAL;
  if (!aligned16(w) || !aligned16(w_packed)) return EQL_EALIGN;
  PackArgs a{};
  a.w = w;
  a.wp = w_packed;
  a.Dp = (int)Dp;
  a.Cp = (int)Cp;
  a.transposed = mode == EQL_PACK_BWDX;
  a.outCh = (int)(a.transposed ? Cp : Dp);
  a.inCh = (int)(a.transposed ? Dp : Cp);
  a.Jin = (int)padded_groups(a.inCh, dtype);
  a.tw = make_twiddles(T);
  const int64_t threads = padded_out(a.outCh) * a.Jin * group_channels(dtype);
  const int64_t grid = ceil_div(threads, 256);
  if (grid > kMaxGrid) return EQL_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(dtype == EQL_F16 ? launch_pack_f16(T, a, (unsigned)grid, s)
                                    : launch_pack_f32(T, a, (unsigned)grid, s));
}

int eqlinear_pack_weight_both(const void* w, void* w_packed, void* w_packed_bwdx, int64_t Dp, int64_t Cp, int T,
                              int dtype, void* stream) {
  int st = check_sizes(0, Cp, Dp, T, dtype);
  if (st != EQL_OK) return st;
  if (!w || !w_packed || !w_packed_bwdx) return EQL_EINVAL;
  if (!aligned16(w) || !aligned16(w_packed) || !aligned16(w_packed_bwdx)) return EQL_EALIGN;
  PackArgs a{};
  a.w = w;
  a.wp = w_packed;
  a.wp2 = w_packed_bwdx;
  a.Dp = (int)Dp;
  a.Cp = (int)Cp;
  a.transposed = 0;
  a.outCh = (int)Dp;
  a.inCh = (int)Cp;
  a.Jin = (int)padded_groups(Cp, dtype);
  a.Jin2 = (int)padded_groups(Dp, dtype);
  a.tw = make_twiddles(T);
  const int64_t g1 = ceil_div(padded_out(Dp) * a.Jin * group_channels(dtype), 256);
  const int64_t g2 = ceil_div(padded_out(Cp) * a.Jin2 * group_channels(dtype), 256);
  if (g1 + g2 > kMaxGrid) return EQL_EINVAL;
  a.blocks1 = (int)g1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(dtype == EQL_F16 ? launch_pack_f16(T, a, (unsigned)(g1 + g2), s)
                                    : launch_pack_f32(T, a, (unsigned)(g1 + g2), s));
}

int eqlinear_fwd(const void* x, const void* w_packed, void* y, int64_t N, int64_t Cp, int64_t Dp,
                 int T, int dtype, void* stream) {
  return run_fwd(x, w_packed, y, N, Cp, Dp, T, dtype, stream);
}

int eqlinear_fwd_fused(const void* x, const void* w_packed, const void* bias, const void* residual,
                       void* y, void* pre_out, int64_t N, int64_t Cp, int64_t Dp, int T, int dtype, int act,
                       void* stream) {
  if (act != EQL_ACT_NONE && act != EQL_ACT_GELU) return EQL_EINVAL;
  int st = check_sizes(N, Cp, Dp, T, dtype);
  if (st != EQL_OK) return st;
  if (N == 0) return EQL_OK;
  if (bias && (reinterpret_cast<uintptr_t>(bias) % (uintptr_t)elt_bytes(dtype)) != 0) return EQL_EALIGN;
  if ((residual && !aligned16(residual)) || (pre_out && !aligned16(pre_out))) return EQL_EALIGN;
  return run_fwd(x, w_packed, y, N, Cp, Dp, T, dtype, stream, true, bias, residual, act, pre_out);
}

size_t eqlinear_fused_epilogue_bwd_workspace_bytes(int64_t N, int64_t Dp, int T, int dtype) {
  if (check_sizes(N, 1, Dp, T, dtype) != EQL_OK || N == 0) return 0;
  return plan_epi(N, Dp, T, dtype).partBytes;
}

int eqlinear_fused_epilogue_bwd(const void* dy, const void* pre, void* dpre, void* dbias, void* workspace,
                                size_t ws_bytes, int64_t N, int64_t Dp, int T, int dtype, int act,
                                void* stream) {
  return epilogue_bwd(dy, pre, dpre, dbias, workspace, ws_bytes, N, Dp, T, dtype, act, stream, false);
}

int eqlinear_fused_epilogue_bwd_noalloc(const void* dy, const void* pre, void* dpre, void* dbias, int64_t N,
                                        int64_t Dp, int T, int dtype, int act, void* stream) {
  return epilogue_bwd(dy, pre, dpre, dbias, nullptr, 0, N, Dp, T, dtype, act, stream, true);
}

int eqlinear_bwd_x(const void* dy, const void* w_packed_bwdx, void* dx, int64_t N, int64_t Cp,
                   int64_t Dp, int T, int dtype, void* stream) {
  // The input gradient is the forward algorithm with the roles of the channel
  // axes swapped: in = D', out = C'.
  int st = check_sizes(N, Cp, Dp, T, dtype);
  if (st != EQL_OK) return st;
  return run_fwd(dy, w_packed_bwdx, dx, N, Dp, Cp, T, dtype, stream);
}

size_t eqlinear_bwd_w_workspace_bytes(int64_t N, int64_t Cp, int64_t Dp, int T, int dtype) {
  if (check_sizes(N, Cp, Dp, T, dtype) != EQL_OK) return 0;
  return plan_bwdw(N, Cp, Dp, T, dtype).total();
}

int eqlinear_bwd_w(const void* x, const void* dy, void* dw, void* workspace, size_t ws_bytes,
                   int64_t N, int64_t Cp, int64_t Dp, int T, int dtype, void* stream) {
  return run_bwdw(x, dy, dw, workspace, ws_bytes, N, Cp, Dp, T, dtype, stream, false);
}

int eqlinear_fwd_train(const void* x, const void* w_packed, void* y, void* workspace, size_t ws_bytes,
                       int64_t N, int64_t Cp, int64_t Dp, int T, int dtype, void* stream) {
  int st = check_sizes(N, Cp, Dp, T, dtype);
  if (st != EQL_OK) return st;
  if (N == 0) return EQL_OK;
  const BwdwPlan p = plan_bwdw(N, Cp, Dp, T, dtype);
  if (!workspace || ws_bytes < p.total()) return EQL_EINVAL;
  if (!aligned16(workspace)) return EQL_EALIGN;
  void* xh = static_cast<char*>(workspace) + p.dyhBytes;
  if (fwd_spec_ok(Cp, T, dtype, p.xhBytes, p.Cpad))
    return run_fwd(x, w_packed, y, N, Cp, Dp, T, dtype, stream, false, nullptr, nullptr, 0, nullptr, xh, p.Cpad,
                   p.xhBytes);
  st = run_fwd(x, w_packed, y, N, Cp, Dp, T, dtype, stream);
  if (st != EQL_OK) return st;
  return run_spec(x, xh, N, Cp, p.Cpad, p.kgCount, T, dtype, static_cast<hipStream_t>(stream));
}

int eqlinear_fwd_fused_train(const void* x, const void* w_packed, const void* bias, const void* residual, void* y,
                             void* pre_out, void* workspace, size_t ws_bytes, int64_t N, int64_t Cp, int64_t Dp, int T,
                             int dtype, int act, void* stream) {
  if (act != EQL_ACT_NONE && act != EQL_ACT_GELU) return EQL_EINVAL;
  int st = check_sizes(N, Cp, Dp, T, dtype);
  if (st != EQL_OK) return st;
  if (N == 0) return EQL_OK;
  const BwdwPlan p = plan_bwdw(N, Cp, Dp, T, dtype);
  if (!workspace || ws_bytes < p.total()) return EQL_EINVAL;
  if (!aligned16(workspace)) return EQL_EALIGN;
  if (bias && (reinterpret_cast<uintptr_t>(bias) % (uintptr_t)elt_bytes(dtype)) != 0) return EQL_EALIGN;
  if ((residual && !aligned16(residual)) || (pre_out && !aligned16(pre_out))) return EQL_EALIGN;
  void* xh = static_cast<char*>(workspace) + p.dyhBytes;
  if (fwd_spec_ok(Cp, T, dtype, p.xhBytes, p.Cpad))
    return run_fwd(x, w_packed, y, N, Cp, Dp, T, dtype, stream, true, bias, residual, act, pre_out, xh, p.Cpad,
                   p.xhBytes);
  st = run_fwd(x, w_packed, y, N, Cp, Dp, T, dtype, stream, true, bias, residual, act, pre_out);
  if (st != EQL_OK) return st;
  return run_spec(x, xh, N, Cp, p.Cpad, p.kgCount, T, dtype, static_cast<hipStream_t>(stream));
}

int eqlinear_bwd_x_train(const void* dy, const void* w_packed_bwdx, void* dx, void* workspace, size_t ws_bytes,
                         int64_t N, int64_t Cp, int64_t Dp, int T, int dtype, void* stream) {
  int st = check_sizes(N, Cp, Dp, T, dtype);
  if (st != EQL_OK) return st;
  if (N == 0) return EQL_OK;
  const BwdwPlan p = plan_bwdw(N, Cp, Dp, T, dtype);
  if (!workspace || ws_bytes < p.total()) return EQL_EINVAL;
  if (!aligned16(workspace)) return EQL_EALIGN;
  // The fused weight-gradient path reads dy itself: nothing to keep.
  if (p.fused) return run_fwd(dy, w_packed_bwdx, dx, N, Dp, Cp, T, dtype, stream);
  if (fwd_spec_ok(Dp, T, dtype, p.dyhBytes, p.Dpad))
    return run_fwd(dy, w_packed_bwdx, dx, N, Dp, Cp, T, dtype, stream, false, nullptr, nullptr, 0, nullptr,
                   workspace, p.Dpad, p.dyhBytes);
  st = run_fwd(dy, w_packed_bwdx, dx, N, Dp, Cp, T, dtype, stream);
  if (st != EQL_OK) return st;
  return run_spec(dy, workspace, N, Dp, p.Dpad, p.kgCount, T, dtype, static_cast<hipStream_t>(stream));
}

int eqlinear_bwd_w_train(const void* dy, void* dw, void* workspace, size_t ws_bytes, int64_t N, int64_t Cp,
                         int64_t Dp, int T, int dtype, void* stream) {
  return run_bwdw(nullptr, dy, dw, workspace, ws_bytes, N, Cp, Dp, T, dtype, stream, true);
}

// p4m (dihedral D4) through the C_4 layer on 2C' x 2D' channels (eql_p4m.h).
static int p4m_map(const void* src, void* dst, int64_t Dp, int64_t Cp, int dtype, void* stream, bool expand) {
  // The C_4 view has 2C' inputs and 2D' outputs of 4 values each: its size rules apply.
  if (Dp < 1 || Cp < 1 || Dp > (INT64_MAX / 4) || Cp > (INT64_MAX / 4)) return EQL_EINVAL;
  const int st = check_sizes(0, 2 * Cp, 2 * Dp, 4, dtype);
  if (st != EQL_OK) return st;
  if (!src || !dst) return EQL_EINVAL;
  if (!aligned16(src) || !aligned16(dst)) return EQL_EALIGN;
  const int64_t grid = ceil_div(Dp * Cp * (expand ? 4 : 8), 256);
  if (grid > kMaxGrid) return EQL_EINVAL;
  P4mArgs a{};
  a.src = src;
  a.dst = dst;
  a.Dp = (int)Dp;
  a.Cp = (int)Cp;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f16 = dtype == EQL_F16;
  return status_of(expand ? launch_p4m_expand(f16, a, (unsigned)grid, s) : launch_p4m_fold(f16, a, (unsigned)grid, s));
}

int eqlinear_p4m_expand_weight(const void* w, void* w_c4, int64_t Dp, int64_t Cp, int dtype, void* stream) {
  return p4m_map(w, w_c4, Dp, Cp, dtype, stream, true);
}

int eqlinear_p4m_fold_weight_grad(const void* dw_c4, void* dw, int64_t Dp, int64_t Cp, int dtype, void* stream) {
  return p4m_map(dw_c4, dw, Dp, Cp, dtype, stream, false);
}

}  // extern "C"
