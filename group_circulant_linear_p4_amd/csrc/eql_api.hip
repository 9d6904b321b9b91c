// C ABI of the EQ-Linear library (declared in include/eqlinear.h): argument
// validation, tile / split policy and launches on the caller's stream.  Nothing
// here allocates device memory or synchronises the host.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

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
  if (N > kMaxN || Cp * T * elt_bytes(dtype) > kMaxRowBytes || Dp * T * elt_bytes(dtype) > kMaxRowBytes)
    return EQL_EINVAL;
  return EQL_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? EQL_OK : EQL_EHIP; }

// Fixed per-stage cost of a forward tile in units of one 32-column block's MFMAs.
constexpr int64_t kFwdStageFixed = 5;

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
int run_fwd(const void* x, const void* wp, void* y, int64_t N, int64_t Cin, int64_t Dout, int T,
            int dtype, void* stream, bool epi = false, const void* bias = nullptr, const void* res = nullptr,
            int act = 0, void* pre = nullptr) {
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
  // barrier, x load and transform measure about five blocks' MFMA time).  Fewest
  // estimated units wins; ties go to the wider tile, which moves fewer bytes per FLOP.
  int nb = 1;
  if (rowsAligned) {
    int64_t best = -1;
    for (int cand = nbm; cand >= 1; cand /= 2) {
      const int64_t rounds = ceil_div(rowTiles * ceil_div(Dout, 32 * cand), (int64_t)cus);
      const int64_t cost = rounds * (kFwdStageFixed + cand);
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
  const int64_t wpBytes = Dout * a.Jpad * 16LL * T;
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
    a.N = (int)rows;
    a.numTiles = (int)(ceil_div(rows, kFwdRows) * colTiles);
    const unsigned grid = (unsigned)std::min<int64_t>(a.numTiles, cus);
    const hipError_t e = epi ? (dtype == EQL_F16 ? launch_fwd_fused_f16(T, nb, a, grid, s)
                                                 : launch_fwd_fused_f32(T, nb, a, grid, s))
                             : (dtype == EQL_F16 ? launch_fwd_f16(T, nb, a, grid, s)
                                                 : launch_fwd_f32(T, nb, a, grid, s));
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
  int DB = 1, CB = 1;  // workgroup tile 64 DB x 64 CB
  int64_t groups = 0, dTiles = 0, cTiles = 0, S = 0, kgPerSplit = 0;
  int64_t items() const { return S * groups * dTiles * cTiles; }
};

// Tile width of one channel axis: 256 unless padding to it adds more than a third
// of the channels, else 64.
int64_t tile_width(int64_t ch) { return ceil_div(ch, 256) * 256 * 3 <= ch * 4 ? 256 : 64; }

struct BwdwPlan {
  int64_t kgCount = 0, Dpad = 0, Cpad = 0;
  GemmPlan real, pair;
  size_t dyhBytes = 0, xhBytes = 0, partRBytes = 0, partPBytes = 0;
  size_t total() const { return dyhBytes + xhBytes + partRBytes + partPBytes; }
};

constexpr int64_t kMinStepsPerSplit = 16;  // keeps partial-spectrum traffic small

// Row ranges (k-step ranges) of one GEMM launch: enough to give every compute unit
// one item.
void plan_splits(GemmPlan& g, int64_t kgCount) {
  const int64_t tiles = g.groups * g.dTiles * g.cTiles;
  if (tiles == 0 || kgCount == 0) return;
  int64_t S = tiles >= kTargetWorkgroups ? 1 : kTargetWorkgroups / tiles;
  S = std::min<int64_t>(S, std::max<int64_t>(1, kgCount / kMinStepsPerSplit));
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
  p.real.groups = nr;
  p.real.dTiles = p.Dpad / wd;
  p.real.cTiles = p.Cpad / wc;
  p.pair.groups = np;
  p.pair.dTiles = p.Dpad / wd;
  p.pair.cTiles = p.Cpad / (64 * p.pair.CB);
  if (N == 0) return p;
  p.kgCount = ceil_div(N, 2 * group_channels(dtype));
  plan_splits(p.real, p.kgCount);
  plan_splits(p.pair, p.kgCount);
  p.dyhBytes = align256((size_t)p.kgCount * T * 2 * (size_t)p.Dpad * 16);
  p.xhBytes = align256((size_t)p.kgCount * T * 2 * (size_t)p.Cpad * 16);
  p.partRBytes = align256((size_t)p.real.S * nr * (size_t)Dp * (size_t)Cp * sizeof(float));
  p.partPBytes = (size_t)p.pair.S * (T - nr) * (size_t)Dp * (size_t)Cp * sizeof(float);
  return p;
}

}  // namespace

extern "C" {

int eqlinear_abi_version(void) { return 101; }

const char* eqlinear_status_string(int status) {
  switch (status) {
    case EQL_OK: return "ok";
    case EQL_EINVAL: return "invalid argument (null pointer, size out of range, unknown dtype or mode, or workspace too small)";
    case EQL_EALIGN: return "a base pointer is not 16-byte aligned";
    case EQL_EUNSUPPORTED: return "group order T above EQL_MAX_T";
    case EQL_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t eqlinear_packed_weight_bytes(int64_t out_ch, int64_t in_ch, int T, int dtype) {
  if (check_sizes(0, in_ch, out_ch, T, dtype) != EQL_OK) return 0;
  return (size_t)out_ch * (size_t)padded_groups(in_ch, dtype) * 16 * T;
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
  const int64_t threads = (int64_t)a.outCh * a.Jin * group_channels(dtype);
  const int64_t grid = ceil_div(threads, 256);
  if (grid > kMaxGrid) return EQL_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return status_of(dtype == EQL_F16 ? launch_pack_f16(T, a, (unsigned)grid, s)
                                    : launch_pack_f32(T, a, (unsigned)grid, s));
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

size_t eqlinear_fused_epilogue_bwd_workspace_bytes(int64_t N, int64_t Dp, int T, int dtype) {
  if (check_sizes(N, 1, Dp, T, dtype) != EQL_OK || N == 0) return 0;
  return plan_epi(N, Dp, T, dtype).partBytes;
}

int eqlinear_fused_epilogue_bwd(const void* dy, const void* pre, void* dpre, void* dbias, void* workspace,
                                size_t ws_bytes, int64_t N, int64_t Dp, int T, int dtype, int act,
                                void* stream) {
  if (act != EQL_ACT_NONE && act != EQL_ACT_GELU) return EQL_EINVAL;
  int st = check_sizes(N, 1, Dp, T, dtype);
  if (st != EQL_OK) return st;
  const EpiPlan p = plan_epi(N, Dp, T, dtype);
  if (p.rowBlocks * p.chunkBlocks > kMaxGrid) return EQL_EINVAL;
  if (N > 0 && (!dy || !dpre || (act == EQL_ACT_GELU && !pre))) return EQL_EINVAL;
  if (dbias && N > 0 && (!workspace || ws_bytes < p.partBytes)) return EQL_EINVAL;
  if ((dy && !aligned16(dy)) || (pre && !aligned16(pre)) || (dpre && !aligned16(dpre)) ||
      (workspace && !aligned16(workspace)) ||
      (dbias && (reinterpret_cast<uintptr_t>(dbias) % (uintptr_t)elt_bytes(dtype)) != 0))
    return EQL_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool f16 = dtype == EQL_F16;
  EpiBwdArgs a{};
  a.dy = dy;
  a.pre = pre;
  a.dpre = dpre;
  a.part = dbias && N > 0 ? static_cast<float*>(workspace) : nullptr;
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
  int st = check_sizes(N, Cp, Dp, T, dtype);
  if (st != EQL_OK) return st;
  const BwdwPlan p = plan_bwdw(N, Cp, Dp, T, dtype);
  if (!dw || (N > 0 && (!x || !dy || !workspace))) return EQL_EINVAL;
  if (ws_bytes < p.total()) return EQL_EINVAL;
  if (!aligned16(dw) || (N > 0 && (!aligned16(x) || !aligned16(dy) || !aligned16(workspace))))
    return EQL_EALIGN;
  const int64_t gdy = ceil_div(p.kgCount * 2 * p.Dpad, 256);
  const int64_t gx = ceil_div(p.kgCount * 2 * p.Cpad, 256);
  const int rwaves = reduce_waves(p.real.S * n_real_planes(T) + p.pair.S * (T - n_real_planes(T)));
  const int64_t rgrid = ceil_div(Dp * Cp, 256 / rwaves);
  if (p.real.items() > kMaxGrid || p.pair.items() > kMaxGrid || gdy > kMaxGrid || gx > kMaxGrid ||
      rgrid > kMaxGrid)
    return EQL_EINVAL;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const Twiddles tw = make_twiddles(T);
  char* ws = static_cast<char*>(workspace);
  float* partR = reinterpret_cast<float*>(ws + p.dyhBytes + p.xhBytes);
  float* partP = reinterpret_cast<float*>(ws + p.dyhBytes + p.xhBytes + p.partRBytes);
  const bool f16 = dtype == EQL_F16;
  if (N > 0) {
    SpecArgs sp{};
    sp.N = (int)N;
    sp.kgCount = (int)p.kgCount;
    sp.tw = tw;
    sp.m = dy;
    sp.out = ws;
    sp.K = (int)Dp;
    sp.Kpad = (int)p.Dpad;
    hipError_t e = f16 ? launch_spec_f16(T, sp, (unsigned)gdy, s) : launch_spec_f32(T, sp, (unsigned)gdy, s);
    if (e != hipSuccess) return EQL_EHIP;
    sp.m = x;
    sp.out = ws + p.dyhBytes;
    sp.K = (int)Cp;
    sp.Kpad = (int)p.Cpad;
    e = f16 ? launch_spec_f16(T, sp, (unsigned)gx, s) : launch_spec_f32(T, sp, (unsigned)gx, s);
    if (e != hipSuccess) return EQL_EHIP;

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
        e = f16 ? launch_bwdw_pair_f16(T, g.DB, g.CB, a, (unsigned)a.numItems, s)
                : launch_bwdw_pair_f32(T, g.DB, g.CB, a, (unsigned)a.numItems, s);
      else
        e = f16 ? launch_bwdw_real_f16(T, g.DB, g.CB, a, (unsigned)a.numItems, s)
                : launch_bwdw_real_f32(T, g.DB, g.CB, a, (unsigned)a.numItems, s);
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

}  // extern "C"
