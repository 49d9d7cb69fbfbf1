// C ABI of the window-attention library: argument validation, workspace sizing, dispatch.
//
// Every check runs on the host before any HIP call, so an invalid call never touches the device.
// Dispatch: bf16 with d == 32 and M <= 32 goes to the MFMA kernels, forward and backward; bf16 with
// d == 64 too, for windows up to 22 x 22 in the forward and 16 x 16 in the backward; grids that M does
// not divide included.  Everything else (float32 tensors, other d, larger windows, the backward of a
// low-rank bias) goes to the float32-arithmetic kernels, which stream the keys through LDS in tiles
// and take any window size up to kMaxWindow.
#include <algorithm>
#include <mutex>

#include "../../include/flashswin.h"
#include "fsw_launch.h"

// Backward scratch for callers that cannot allocate (flashswin_wattn_bwd_noalloc): one fixed array
// per GPU, which that GPU holds until the process ends.  Host code never passes `scratch` itself to
// a kernel (on the host it names a stand-in, not the device array); it passes the device address
// that hipGetSymbolAddress returned for the current device.
static __device__ __align__(256) unsigned char scratch[FLASHSWIN_SCRATCH_BYTES];

namespace {

constexpr int kMaxM = 32;        // largest window of the MFMA kernels
constexpr int kMaxWindow = 128;  // largest window of any kernel (N = 16384 tokens)

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_d(int d) { return d == 8 || d == 16 || d == 32 || d == 64; }

// Shape rules shared by forward, backward and workspace sizing.  Fills g on success.
int check_shape(int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M, int shift, int dtype, fsw::Geom* g) {
  if (B < 0 || Hg < 1 || Wg < 1 || heads < 1 || M < 1 || d < 1) return FSW_ERR_INVALID_ARG;
  if (shift < 0 || shift >= M) return FSW_ERR_INVALID_ARG;
  if (d % 4 != 0) return FSW_ERR_INVALID_ARG;
  if (dtype != FSW_F32 && dtype != FSW_BF16) return FSW_ERR_INVALID_ARG;
  if (!supported_d(d) || M > kMaxWindow) return FSW_ERR_UNSUPPORTED;
  // int32 grid coordinates and int64 element offsets: keep every product well inside int64,
  // and the flat 1-D launch grid inside 2^31 workgroups.
  const int64_t lim = (int64_t)1 << 30;
  if (Hg > lim || Wg > lim || heads > (1 << 20)) return FSW_ERR_UNSUPPORTED;
  const long double elems = (long double)B * Hg * Wg * heads * d;
  if (elems > (long double)((int64_t)1 << 56)) return FSW_ERR_UNSUPPORTED;
  // a grid that M does not divide is padded to the next multiples of M (see fsw::Geom)
  const int64_t nH = (Hg + M - 1) / M, nW = (Wg + M - 1) / M;
  const long double wgs = (long double)B * nH * nW * heads * 8;
  if (wgs > (long double)((int64_t)1 << 31) - 1) return FSW_ERR_UNSUPPORTED;
  g->B = B;
  g->Hg = (int)Hg;
  g->Wg = (int)Wg;
  g->heads = heads;
  g->d = d;
  g->M = M;
  g->shift = shift;
  g->nH = (int)nH;
  g->nW = (int)nW;
  g->Hp = (int)(nH * M);
  g->Wp = (int)(nW * M);
  g->N = M * M;
  g->xs = (int64_t)heads * d;
  g->os = (int64_t)heads * d;
  return FSW_OK;
}

size_t elem_bytes(int dtype) { return dtype == FSW_BF16 ? 2 : 4; }

// Byte ranges [a, a + na) and [b, b + nb) overlap (a null or empty range overlaps nothing).
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// A buffer and its size in bytes.
struct Span {
  const void* p;
  size_t n;
};
// Every output span is disjoint from every input span and from the other outputs.  Inputs may
// share memory with each other (they are only read).
template <size_t NO, size_t NI>
bool outputs_disjoint(const Span (&outs)[NO], const Span (&ins)[NI]) {
  for (size_t i = 0; i < NO; ++i) {
    for (size_t j = 0; j < NI; ++j)
      if (overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return false;
    for (size_t j = i + 1; j < NO; ++j)
      if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return false;
  }
  return true;
}

// Bytes of one token-grid tensor, of LSE and of one theta table of geometry g.
struct Sizes {
  size_t tens, lse, theta;
};
Sizes sizes_of(const fsw::Geom& g, int dtype) {
  const size_t tokens = (size_t)(g.B * g.Hg * g.Wg);
  return {tokens * (size_t)g.os * elem_bytes(dtype), tokens * (size_t)g.heads * 4,
          (size_t)g.heads * (size_t)(g.d / 4) * 4};
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t delta_off, scal_off, partials_off, lr_off, total;
  int64_t n_partials;
};

// Kernel family of a backward call.
enum class BwdPath { kScalar, kMfma32, kMfma64, kMfmaLowRank };

// rank > 0: room for the per-window gradients of both low-rank bias factors.
WsLayout workspace_layout(const fsw::Geom& g, BwdPath path, int rank = 0) {
  WsLayout w;
  const int64_t rows = g.B * g.Hg * g.Wg * g.heads;
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  w.delta_off = 0;
  w.scal_off = align256((size_t)rows * sizeof(float));
  w.partials_off = w.scal_off + align256((size_t)nwh * 4 * sizeof(float));
  w.n_partials = path == BwdPath::kMfma32 ? fsw::bwd_mfma_partials(g)
                 : path == BwdPath::kMfma64 || path == BwdPath::kMfmaLowRank ? fsw::bwd_window_partials(g)
                                                                             : fsw::bwd_scalar_partials(g);
  w.lr_off = w.partials_off + align256((size_t)w.n_partials * (g.d / 2) * sizeof(float));
  const int64_t lr_floats = 2 * g.B * g.nH * g.nW * g.heads * g.N * rank +
                            (path == BwdPath::kMfmaLowRank ? fsw::lowrank_mfma_extra_floats(g) : 0);
  w.total = w.lr_off + align256((size_t)lr_floats * sizeof(float));
  return w;
}

// Padded grids: padding tokens are skipped by every kernel family except the materialized comparison
// and the M = 8 forward variant.
bool padded(const fsw::Geom& g) { return g.Hp != g.Hg || g.Wp != g.Wg; }
bool use_mfma_fwd(const fsw::Geom& g, int dtype) { return dtype == FSW_BF16 && fsw::fwd_mfma_supported(g); }
// A low-rank bias runs on the whole-window MFMA kernels where they serve the shape, else on the
// float32-arithmetic kernels.
BwdPath bwd_path(const fsw::Geom& g, int dtype, int rank = 0) {
  if (rank > 0)
    return dtype == FSW_BF16 && fsw::bwd_lowrank_mfma_supported(g, rank) ? BwdPath::kMfmaLowRank : BwdPath::kScalar;
  if (dtype != FSW_BF16) return BwdPath::kScalar;
  if (fsw::kHaveMfmaBwd && g.d == 32 && g.M <= kMaxM) return BwdPath::kMfma32;
  if (fsw::bwd_d64_supported(g)) return BwdPath::kMfma64;
  return BwdPath::kScalar;
}

// Pointer checks and dispatch of a forward whose shape (and q/k/v token stride) is in g.
// stats (optional): the backward's operand maxima, from the MFMA forward itself or from a kernel of
// their own after the float32-arithmetic forward (bf16, d 32 or 64; other shapes leave them unwritten:
// no backward reads them).
int fwd_impl(const void* q, const void* k, const void* v, const float* theta_row, const float* theta_col, void* out,
             float* lse, const fsw::Geom& g, int dtype, void* hip_stream, const fsw::LowRank& lr = {},
             float* stats = nullptr) {
  if (!q || !k || !v || !out || !theta_row || !theta_col) return FSW_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FSW_ERR_INVALID_ARG;
  if (!aligned(theta_row, 4) || !aligned(theta_col, 4) || (lse && !aligned(lse, 4))) return FSW_ERR_INVALID_ARG;
  fsw::FwdArgs a{q, k, v, theta_row, theta_col, out, lse, g, dtype, lr};
  a.stats = stats;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  const bool mfma = lr.rank == 0 ? use_mfma_fwd(g, dtype)
                                  : dtype == FSW_BF16 && fsw::fwd_mfma_lowrank_supported(g, lr.rank);
  hipError_t e = mfma ? fsw::launch_fwd_mfma(a, s) : fsw::launch_fwd_scalar(a, s);
  if (e == hipSuccess && stats && !mfma && dtype == FSW_BF16 && (g.d == 32 || g.d == 64))
    e = fsw::launch_operand_maxima(a, s);
  return e == hipSuccess ? FSW_OK : FSW_ERR_HIP;
}

// Null and alignment checks of a backward's tensor pointers.
bool bwd_pointers_ok(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                     const float* theta_row, const float* theta_col, void* dq, void* dk, void* dv, float* dtheta_row,
                     float* dtheta_col) {
  const void* ptrs16[] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* p : ptrs16)
    if (!p || !aligned(p, 16)) return false;
  const void* ptrs4[] = {lse, theta_row, theta_col, dtheta_row, dtheta_col};
  for (const void* p : ptrs4)
    if (!p || !aligned(p, 4)) return false;
  return dtheta_row != dtheta_col;
}

// Pointer, workspace checks and dispatch of a backward whose shape (and strides) is in g.
int bwd_impl(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
             const float* theta_row, const float* theta_col, void* dq, void* dk, void* dv, float* dtheta_row,
             float* dtheta_col, void* workspace, size_t workspace_bytes, const fsw::Geom& g, int dtype,
             void* hip_stream, const fsw::LowRank& lr = {}, float* du = nullptr, float* dw = nullptr,
             const float* stats = nullptr) {
  if (!bwd_pointers_ok(q, k, v, out, dout, lse, theta_row, theta_col, dq, dk, dv, dtheta_row, dtheta_col))
    return FSW_ERR_INVALID_ARG;
  const BwdPath path = bwd_path(g, dtype, lr.rank);
  const WsLayout ws = workspace_layout(g, path, lr.rank);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < ws.total) return FSW_ERR_WORKSPACE;
  char* base = static_cast<char*>(workspace);
  fsw::BwdArgs a{q,  k,  v,          out,        dout, lse, theta_row, theta_col,
                 dq, dk, dv,         dtheta_row, dtheta_col, g, dtype,
                 reinterpret_cast<float*>(base + ws.delta_off), reinterpret_cast<float*>(base + ws.scal_off),
                 reinterpret_cast<float*>(base + ws.partials_off), ws.n_partials, lr, du, dw,
                 reinterpret_cast<float*>(base + ws.lr_off)};
  a.stats = stats;
  hipStream_t s = reinterpret_cast<hipStream_t>(hip_stream);
  const hipError_t e = path == BwdPath::kMfma32         ? fsw::launch_bwd_mfma(a, s)
                       : path == BwdPath::kMfma64       ? fsw::launch_bwd_d64(a, s)
                       : path == BwdPath::kMfmaLowRank  ? fsw::launch_bwd_lowrank_mfma(a, s)
                                                        : fsw::launch_bwd_scalar(a, s);
  return e == hipSuccess ? FSW_OK : FSW_ERR_HIP;
}

// Device address of `scratch` on the current device, looked up once per device; nullptr (and the
// HIP error in *err) when the lookup fails.
constexpr int kMaxScratchDevices = 64;

void* scratch_address(hipError_t* err) {
  static std::once_flag once[kMaxScratchDevices];
  static void* addr[kMaxScratchDevices];
  static hipError_t status[kMaxScratchDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    addr[dev] = status[dev] == hipSuccess ? p : nullptr;
  });
  *err = status[dev];
  return addr[dev];
}

}  // namespace

extern "C" {

int flashswin_version(void) { return 102; }

const char* flashswin_status_string(int status) {
  switch (status) {
    case FSW_OK: return "FSW_OK";
    case FSW_ERR_INVALID_ARG: return "FSW_ERR_INVALID_ARG: invalid shape, pointer, alignment, shift or dtype";
    case FSW_ERR_UNSUPPORTED: return "FSW_ERR_UNSUPPORTED: valid arguments this library does not implement";
    case FSW_ERR_WORKSPACE: return "FSW_ERR_WORKSPACE: workspace missing or too small";
    case FSW_ERR_HIP: return "FSW_ERR_HIP: a HIP kernel launch failed";
    case FSW_ERR_SCRATCH:
      return "FSW_ERR_SCRATCH: the backward needs more workspace than the library's fixed scratch array "
             "(FLASHSWIN_SCRATCH_BYTES) holds; call flashswin_wattn_bwd with a caller workspace";
    default: return "unknown flashswin status";
  }
}

int flashswin_wattn_fwd(const void* q, const void* k, const void* v, const float* theta_row, const float* theta_col,
                        void* out, float* lse, int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M, int shift,
                        int dtype, void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  const Sizes z = sizes_of(g, dtype);
  const Span outs[] = {{out, z.tens}, {lse, z.lse}};
  const Span ins[] = {{q, z.tens}, {k, z.tens}, {v, z.tens}, {theta_row, z.theta}, {theta_col, z.theta}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  return fwd_impl(q, k, v, theta_row, theta_col, out, lse, g, dtype, hip_stream);
}

// The packed forward, with the operand summary when stats is non-null.
static int fwd_packed_impl(const void* qkv, const float* theta_row, const float* theta_col, void* out, float* lse,
                           float* stats, bool with_stats, int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M,
                           int shift, int dtype, void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  if ((long double)B * Hg * Wg * 3 * heads * d > (long double)((int64_t)1 << 56)) return FSW_ERR_UNSUPPORTED;
  if (!qkv) return FSW_ERR_INVALID_ARG;
  if (with_stats && (!stats || !aligned(stats, 4))) return FSW_ERR_INVALID_ARG;
  const size_t eb = elem_bytes(dtype);
  const Sizes z = sizes_of(g, dtype);
  const size_t sb = with_stats ? (size_t)(g.B * g.nH * g.nW * g.heads) * 4 * sizeof(float) : 0;
  const Span outs[] = {{out, z.tens}, {lse, z.lse}, {stats, sb}};
  const Span ins[] = {{qkv, 3 * z.tens}, {theta_row, z.theta}, {theta_col, z.theta}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  g.xs = 3 * g.os;
  const char* base = static_cast<const char*>(qkv);
  const size_t slot = (size_t)g.os * eb;  // bytes from q to k and from k to v within a token
  return fwd_impl(base, base + slot, base + 2 * slot, theta_row, theta_col, out, lse, g, dtype, hip_stream, {},
                  with_stats ? stats : nullptr);
}

int flashswin_wattn_fwd_packed(const void* qkv, const float* theta_row, const float* theta_col, void* out, float* lse,
                               int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M, int shift, int dtype,
                               void* hip_stream) {
  return fwd_packed_impl(qkv, theta_row, theta_col, out, lse, nullptr, false, B, Hg, Wg, heads, d, M, shift, dtype,
                         hip_stream);
}

int flashswin_wattn_fwd_packed_stats(const void* qkv, const float* theta_row, const float* theta_col, void* out,
                                     float* lse, float* stats, int64_t B, int64_t Hg, int64_t Wg, int heads, int d,
                                     int M, int shift, int dtype, void* hip_stream) {
  return fwd_packed_impl(qkv, theta_row, theta_col, out, lse, stats, true, B, Hg, Wg, heads, d, M, shift, dtype,
                         hip_stream);
}

size_t flashswin_wattn_bwd_workspace_size(int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M, int shift,
                                          int dtype) {
  fsw::Geom g;
  if (check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g) != FSW_OK) return 0;
  if (B == 0) return 0;
  return workspace_layout(g, bwd_path(g, dtype)).total;
}

int flashswin_wattn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                        const float* lse, const float* theta_row, const float* theta_col, void* dq, void* dk, void* dv,
                        float* dtheta_row, float* dtheta_col, void* workspace, size_t workspace_bytes, int64_t B,
                        int64_t Hg, int64_t Wg, int heads, int d, int M, int shift, int dtype, void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  const Sizes z = sizes_of(g, dtype);
  const Span outs[] = {{dq, z.tens},         {dk, z.tens},          {dv, z.tens},
                       {dtheta_row, z.theta}, {dtheta_col, z.theta}, {workspace, workspace_bytes}};
  const Span ins[] = {{q, z.tens},   {k, z.tens},           {v, z.tens},          {out, z.tens},
                      {dout, z.tens}, {lse, z.lse}, {theta_row, z.theta}, {theta_col, z.theta}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  return bwd_impl(q, k, v, out, dout, lse, theta_row, theta_col, dq, dk, dv, dtheta_row, dtheta_col, workspace,
                  workspace_bytes, g, dtype, hip_stream);
}

// The packed backward, taking the forward's operand summary when stats is non-null.
static int bwd_packed_impl(const void* qkv, const void* out, const void* dout, const float* lse,
                           const float* theta_row, const float* theta_col, const float* stats, bool with_stats,
                           void* dqkv, float* dtheta_row, float* dtheta_col, void* workspace, size_t workspace_bytes,
                           int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M, int shift, int dtype,
                           void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  if ((long double)B * Hg * Wg * 3 * heads * d > (long double)((int64_t)1 << 56)) return FSW_ERR_UNSUPPORTED;
  if (!qkv || !dqkv) return FSW_ERR_INVALID_ARG;
  if (with_stats && (!stats || !aligned(stats, 4))) return FSW_ERR_INVALID_ARG;
  const size_t eb = elem_bytes(dtype);
  const Sizes z = sizes_of(g, dtype);
  const size_t sb = with_stats ? (size_t)(g.B * g.nH * g.nW * g.heads) * 4 * sizeof(float) : 0;
  const Span outs[] = {{dqkv, 3 * z.tens}, {dtheta_row, z.theta}, {dtheta_col, z.theta},
                       {workspace, workspace_bytes}};
  const Span ins[] = {{qkv, 3 * z.tens}, {out, z.tens}, {dout, z.tens}, {lse, z.lse}, {theta_row, z.theta},
                      {theta_col, z.theta}, {stats, sb}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  g.xs = 3 * g.os;
  const size_t slot = (size_t)g.os * eb;
  const char* x = static_cast<const char*>(qkv);
  char* dx = static_cast<char*>(dqkv);
  return bwd_impl(x, x + slot, x + 2 * slot, out, dout, lse, theta_row, theta_col, dx, dx + slot, dx + 2 * slot,
                  dtheta_row, dtheta_col, workspace, workspace_bytes, g, dtype, hip_stream, {}, nullptr, nullptr,
                  with_stats ? stats : nullptr);
}

int flashswin_wattn_bwd_packed(const void* qkv, const void* out, const void* dout, const float* lse,
                               const float* theta_row, const float* theta_col, void* dqkv, float* dtheta_row,
                               float* dtheta_col, void* workspace, size_t workspace_bytes, int64_t B, int64_t Hg,
                               int64_t Wg, int heads, int d, int M, int shift, int dtype, void* hip_stream) {
  return bwd_packed_impl(qkv, out, dout, lse, theta_row, theta_col, nullptr, false, dqkv, dtheta_row, dtheta_col,
                         workspace, workspace_bytes, B, Hg, Wg, heads, d, M, shift, dtype, hip_stream);
}

int flashswin_wattn_bwd_packed_stats(const void* qkv, const void* out, const void* dout, const float* lse,
                                     const float* theta_row, const float* theta_col, const float* stats, void* dqkv,
                                     float* dtheta_row, float* dtheta_col, void* workspace, size_t workspace_bytes,
                                     int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M, int shift, int dtype,
                                     void* hip_stream) {
  return bwd_packed_impl(qkv, out, dout, lse, theta_row, theta_col, stats, true, dqkv, dtheta_row, dtheta_col,
                         workspace, workspace_bytes, B, Hg, Wg, heads, d, M, shift, dtype, hip_stream);
}

// Low-rank bias factors of a call: rank in [1, kMaxRank], U and W non-null and 4-byte aligned.
static_assert(fsw::kMaxRank == FLASHSWIN_MAX_RANK, "rank limit of the kernels and of the header");
static int check_lowrank(const float* u, const float* w, int rank) {
  if (rank < 1) return FSW_ERR_INVALID_ARG;
  if (rank > fsw::kMaxRank) return FSW_ERR_UNSUPPORTED;
  if (!u || !w || !aligned(u, 4) || !aligned(w, 4)) return FSW_ERR_INVALID_ARG;
  return FSW_OK;
}

static size_t factor_bytes(const fsw::Geom& g, int rank) { return (size_t)g.heads * g.N * rank * sizeof(float); }

int flashswin_wattn_fwd_lowrank(const void* q, const void* k, const void* v, const float* theta_row,
                                const float* theta_col, const float* bias_u, const float* bias_w, int rank, void* out,
                                float* lse, int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M, int shift,
                                int dtype, void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if ((st = check_lowrank(bias_u, bias_w, rank)) != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  const Sizes z = sizes_of(g, dtype);
  const size_t fb = factor_bytes(g, rank);
  const Span outs[] = {{out, z.tens}, {lse, z.lse}};
  const Span ins[] = {{q, z.tens}, {k, z.tens}, {v, z.tens}, {theta_row, z.theta}, {theta_col, z.theta},
                      {bias_u, fb}, {bias_w, fb}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  fsw::LowRank lr;
  lr.u = bias_u;
  lr.w = bias_w;
  lr.rank = rank;
  return fwd_impl(q, k, v, theta_row, theta_col, out, lse, g, dtype, hip_stream, lr);
}

size_t flashswin_wattn_bwd_lowrank_workspace_size(int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M,
                                                  int shift, int dtype, int rank) {
  fsw::Geom g;
  if (check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g) != FSW_OK) return 0;
  if (B == 0 || rank < 1 || rank > fsw::kMaxRank) return 0;
  return workspace_layout(g, bwd_path(g, dtype, rank), rank).total;
}

int flashswin_wattn_bwd_lowrank(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                const float* lse, const float* theta_row, const float* theta_col,
                                const float* bias_u, const float* bias_w, int rank, void* dq, void* dk, void* dv,
                                float* dtheta_row, float* dtheta_col, float* dbias_u, float* dbias_w,
                                void* workspace, size_t workspace_bytes, int64_t B, int64_t Hg, int64_t Wg, int heads,
                                int d, int M, int shift, int dtype, void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if ((st = check_lowrank(bias_u, bias_w, rank)) != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  if (!dbias_u || !dbias_w || !aligned(dbias_u, 4) || !aligned(dbias_w, 4)) return FSW_ERR_INVALID_ARG;
  const Sizes z = sizes_of(g, dtype);
  const size_t fb = factor_bytes(g, rank);
  const Span outs[] = {{dq, z.tens},         {dk, z.tens},          {dv, z.tens}, {dtheta_row, z.theta},
                       {dtheta_col, z.theta}, {dbias_u, fb}, {dbias_w, fb}, {workspace, workspace_bytes}};
  const Span ins[] = {{q, z.tens},    {k, z.tens},   {v, z.tens},          {out, z.tens},        {dout, z.tens},
                      {lse, z.lse},   {bias_u, fb},  {bias_w, fb},         {theta_row, z.theta}, {theta_col, z.theta}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  fsw::LowRank lr;
  lr.u = bias_u;
  lr.w = bias_w;
  lr.rank = rank;
  return bwd_impl(q, k, v, out, dout, lse, theta_row, theta_col, dq, dk, dv, dtheta_row, dtheta_col, workspace,
                  workspace_bytes, g, dtype, hip_stream, lr, dbias_u, dbias_w);
}

size_t flashswin_wattn_fwd_materialized_workspace_size(int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M,
                                                       int shift, int dtype) {
  fsw::Geom g;
  if (check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g) != FSW_OK) return 0;
  if (B == 0 || dtype != FSW_BF16 || d != 32 || M > kMaxM || padded(g)) return 0;
  return fsw::materialized_workspace_bytes(g);
}

int flashswin_wattn_fwd_materialized(const void* q, const void* k, const void* v, const float* theta_row,
                                     const float* theta_col, const float* bias, void* out, float* lse,
                                     void* workspace, size_t workspace_bytes, int64_t B, int64_t Hg, int64_t Wg,
                                     int heads, int d, int M, int shift, int dtype, void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if (dtype != FSW_BF16 || d != 32 || M > kMaxM || padded(g)) return FSW_ERR_UNSUPPORTED;
  if (B == 0) return FSW_OK;
  if (!q || !k || !v || !out || !theta_row || !theta_col) return FSW_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FSW_ERR_INVALID_ARG;
  if (!aligned(theta_row, 4) || !aligned(theta_col, 4) || (lse && !aligned(lse, 4)) || (bias && !aligned(bias, 4)))
    return FSW_ERR_INVALID_ARG;
  const size_t need = fsw::materialized_workspace_bytes(g);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return FSW_ERR_WORKSPACE;
  const Sizes z = sizes_of(g, dtype);
  const size_t bias_bytes = (size_t)heads * (2 * M - 1) * (2 * M - 1) * sizeof(float);
  const Span outs[] = {{out, z.tens}, {lse, z.lse}, {workspace, need}};
  const Span ins[] = {{q, z.tens},          {k, z.tens},          {v, z.tens},
                      {theta_row, z.theta}, {theta_col, z.theta}, {bias, bias ? bias_bytes : 0}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  fsw::FwdArgs a{q, k, v, theta_row, theta_col, out, lse, g, dtype};
  const hipError_t e = fsw::launch_fwd_materialized(a, bias, workspace, reinterpret_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? FSW_OK : FSW_ERR_HIP;
}

size_t flashswin_wattn_stats_bytes(int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M, int shift, int dtype) {
  fsw::Geom g;
  if (check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g) != FSW_OK) return 0;
  return (size_t)(g.B * g.nH * g.nW * g.heads) * 4 * sizeof(float);
}

int flashswin_wattn_fwd_stats(const void* q, const void* k, const void* v, const float* theta_row,
                              const float* theta_col, const float* bias_u, const float* bias_w, int rank, void* out,
                              float* lse, float* stats, int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M,
                              int shift, int dtype, void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if (rank != 0 && (st = check_lowrank(bias_u, bias_w, rank)) != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  if (!stats || !aligned(stats, 4)) return FSW_ERR_INVALID_ARG;
  const Sizes z = sizes_of(g, dtype);
  const size_t fb = rank > 0 ? factor_bytes(g, rank) : 0;
  const size_t sb = (size_t)(g.B * g.nH * g.nW * g.heads) * 4 * sizeof(float);
  const Span outs[] = {{out, z.tens}, {lse, z.lse}, {stats, sb}};
  const Span ins[] = {{q, z.tens}, {k, z.tens}, {v, z.tens}, {theta_row, z.theta}, {theta_col, z.theta},
                      {bias_u, fb}, {bias_w, fb}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  fsw::LowRank lr;
  if (rank > 0) {
    lr.u = bias_u;
    lr.w = bias_w;
    lr.rank = rank;
  }
  return fwd_impl(q, k, v, theta_row, theta_col, out, lse, g, dtype, hip_stream, lr, stats);
}

int flashswin_wattn_bwd_stats(const void* q, const void* k, const void* v, const void* out, const void* dout,
                              const float* lse, const float* theta_row, const float* theta_col, const float* bias_u,
                              const float* bias_w, int rank, const float* stats, void* dq, void* dk, void* dv,
                              float* dtheta_row, float* dtheta_col, float* dbias_u, float* dbias_w, void* workspace,
                              size_t workspace_bytes, int64_t B, int64_t Hg, int64_t Wg, int heads, int d, int M,
                              int shift, int dtype, void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if (rank != 0 && (st = check_lowrank(bias_u, bias_w, rank)) != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  if (!stats || !aligned(stats, 4)) return FSW_ERR_INVALID_ARG;
  if (rank > 0 && (!dbias_u || !dbias_w || !aligned(dbias_u, 4) || !aligned(dbias_w, 4))) return FSW_ERR_INVALID_ARG;
  const Sizes z = sizes_of(g, dtype);
  const size_t fb = rank > 0 ? factor_bytes(g, rank) : 0;
  const size_t sb = (size_t)(g.B * g.nH * g.nW * g.heads) * 4 * sizeof(float);
  const Span outs[] = {{dq, z.tens},         {dk, z.tens},          {dv, z.tens},
                       {dtheta_row, z.theta}, {dtheta_col, z.theta}, {dbias_u, fb},
                       {dbias_w, fb},         {workspace, workspace_bytes}};
  const Span ins[] = {{q, z.tens},    {k, z.tens},  {v, z.tens},   {out, z.tens},        {dout, z.tens},
                      {lse, z.lse},   {bias_u, fb}, {bias_w, fb},  {theta_row, z.theta}, {theta_col, z.theta},
                      {stats, sb}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  fsw::LowRank lr;
  if (rank > 0) {
    lr.u = bias_u;
    lr.w = bias_w;
    lr.rank = rank;
  }
  return bwd_impl(q, k, v, out, dout, lse, theta_row, theta_col, dq, dk, dv, dtheta_row, dtheta_col, workspace,
                  workspace_bytes, g, dtype, hip_stream, lr, rank > 0 ? dbias_u : nullptr,
                  rank > 0 ? dbias_w : nullptr, stats);
}

int flashswin_wattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                const float* lse, const float* theta_row, const float* theta_col, void* dq, void* dk,
                                void* dv, float* dtheta_row, float* dtheta_col, int64_t B, int64_t Hg, int64_t Wg,
                                int heads, int d, int M, int shift, int dtype, void* hip_stream) {
  fsw::Geom g;
  int st = check_shape(B, Hg, Wg, heads, d, M, shift, dtype, &g);
  if (st != FSW_OK) return st;
  if (B == 0) return FSW_OK;
  // the size limit is checked before any HIP call
  const size_t need = workspace_layout(g, bwd_path(g, dtype)).total;
  if (need > (size_t)FLASHSWIN_SCRATCH_BYTES) return FSW_ERR_SCRATCH;
  const Sizes z = sizes_of(g, dtype);
  const Span outs[] = {{dq, z.tens}, {dk, z.tens}, {dv, z.tens}, {dtheta_row, z.theta}, {dtheta_col, z.theta}};
  const Span ins[] = {{q, z.tens},   {k, z.tens},           {v, z.tens},          {out, z.tens},
                      {dout, z.tens}, {lse, z.lse}, {theta_row, z.theta}, {theta_col, z.theta}};
  if (!outputs_disjoint(outs, ins)) return FSW_ERR_INVALID_ARG;
  if (!bwd_pointers_ok(q, k, v, out, dout, lse, theta_row, theta_col, dq, dk, dv, dtheta_row, dtheta_col))
    return FSW_ERR_INVALID_ARG;
  hipError_t e = hipSuccess;
  void* ws = scratch_address(&e);
  if (!ws) return FSW_ERR_HIP;
  // every section of the workspace is written before it is read (Delta and the window maxima by
  // the prologue, each dtheta partial row by its workgroup), so nothing needs clearing first
  return bwd_impl(q, k, v, out, dout, lse, theta_row, theta_col, dq, dk, dv, dtheta_row, dtheta_col, ws,
                  (size_t)FLASHSWIN_SCRATCH_BYTES, g, dtype, hip_stream);
}

}  // extern "C"
