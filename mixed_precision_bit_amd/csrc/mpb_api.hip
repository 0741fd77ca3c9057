// libmpb host side: argument validation, the host mirror of the weight page
// table, workspace layout and launch sequencing. Every export validates on the
// host before enqueuing anything and never lets a C++ exception escape.
#include <algorithm>
#include <string>
#include <vector>

#include "mpb.h"
#include "mpb_device.h"
#include "mpb_internal.h"

// Workspace of moe_ffn_static, for callers that cannot allocate: a file-scope
// device array, one copy per GPU, held until the process ends. Host code only
// ever uses the address hipGetSymbolAddress returns for the current device,
// never the array's name (which on the host is a stand-in, not a device
// address).
static constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// One page transfer of a block: planes lo..hi-1 move to the GPU (dir 1) or to
// the CPU (dir 2); done once ev, recorded on the copy stream after the copies,
// has completed.
struct Xfer {
  hipEvent_t ev = nullptr;
  int dir = 0, lo = 0, hi = 0;
};

struct State {
  bool init = false;
  int H = 0, I = 0, E = 0, S = 0, K = 0;
  int32_t* q_dev = nullptr;
  std::vector<int> q;         // host mirror of committed bitwidths
  std::vector<int> resident;  // planes 0..resident-1 of each block are GPU-resident
  std::vector<Xfer> xfer;     // the block's page transfer, if one has been enqueued
  // recorded on the bound stream each time q_i is lowered: every launch that
  // may read a plane above the new q_i was enqueued before it
  std::vector<hipEvent_t> lower_ev;
  hipStream_t stream = nullptr;
  int nb() const { return 2 * (E + S); }
};

State g;
thread_local std::string g_err;

// Per-device address of the scratch array (below), resolved with the device
// current; null until then.
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipEvent_t g_ev[7];
int g_nev = 0;

void mark(int k, hipStream_t s) {
  if (g_nev >= 5) (void)hipEventRecord(g_ev[k], s);
}

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MPB_E_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

// Address of this device's scratch array, resolved once per device (with the
// device current). Returns MPB_OK or an error code.
int resolve_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "scratch: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MPB_E_HIP, "scratch: device index above 63");
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "scratch: hipGetSymbolAddress");
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return MPB_OK;
}

void block_shape(int i, int* N, int* Kd) {
  if (i % 2 == 0) { *N = 2 * g.I; *Kd = g.H; }
  else { *N = g.H; *Kd = g.I; }
}

int64_t block_bytes(int N, int Kd, int b) {
  return (int64_t)N * Kd * b / 8 + (int64_t)N * (1 << b) * 2;
}

// Moves a finished transfer's pages to their new state. Returns MPB_OK, or
// MPB_E_HIP if the copy stream reported an error.
int refresh_xfer(int i) {
  Xfer& x = g.xfer[i];
  if (!x.dir) return MPB_OK;
  const hipError_t e = hipEventQuery(x.ev);
  if (e == hipErrorNotReady) return MPB_OK;
  if (e != hipSuccess) return hip_fail(e, "page transfer");
  if (x.dir == 1) g.resident[i] = x.hi;
  x.dir = 0;
  return MPB_OK;
}

// Enqueues the copies of pages lo..hi-1 of block i: page p is plane page p
// and, from p = 2 on, the table image of bitwidth p + 1 (the table a block
// needs once it reads p + 1 planes).
int copy_pages(int i, int lo, int hi, void* const* host_planes, uint32_t* const* dev_planes,
               void* const* host_tables, uint16_t* const* dev_tables, bool to_gpu, hipStream_t cs) {
  int N, Kd;
  block_shape(i, &N, &Kd);
  const size_t pbytes = (size_t)N * mpb::page_chunks(Kd) * 16;
  Xfer& x = g.xfer[i];
  hipError_t e = hipSuccess;
  if (!x.ev) e = hipEventCreateWithFlags(&x.ev, hipEventDisableTiming);
  for (int p = lo; e == hipSuccess && p < hi; ++p) {
    e = to_gpu ? hipMemcpyAsync(dev_planes[p], host_planes[p], pbytes, hipMemcpyHostToDevice, cs)
               : hipMemcpyAsync(host_planes[p], dev_planes[p], pbytes, hipMemcpyDeviceToHost, cs);
    const int t = p - 2;  // table image of bitwidth p + 1, entry (p + 1) - 3
    if (e == hipSuccess && t >= 0) {
      const size_t tbytes = (size_t)((N + 127) / 128) * (256u << (p + 1));
      e = to_gpu ? hipMemcpyAsync(dev_tables[t], host_tables[t], tbytes, hipMemcpyHostToDevice, cs)
                 : hipMemcpyAsync(host_tables[t], dev_tables[t], tbytes, hipMemcpyDeviceToHost, cs);
    }
  }
  if (e == hipSuccess) e = hipEventRecord(x.ev, cs);
  if (e != hipSuccess) return hip_fail(e, to_gpu ? "mpb_reload_pages" : "mpb_offload_pages");
  x.dir = to_gpu ? 1 : 2;
  x.lo = lo;
  x.hi = hi;
  return MPB_OK;
}

// Checks the pointers of pages lo..hi-1 (plane p, and table p - 2 from p = 3 on).
bool page_ptrs_ok(int lo, int hi, const void* const* hp, const void* const* dp, const void* const* ht,
                  const void* const* dt) {
  if (!hp || !dp || !ht || !dt) return false;
  for (int p = lo; p < hi; ++p)
    if (!hp[p] || !dp[p] || !ht[p - 2] || !dt[p - 2]) return false;
  return true;
}

}  // namespace

namespace mpb {

int set_error(int code, const char* msg) { return fail(code, msg); }

bool geometry_ok(int H, int I, int E, int S, int K, const char** why) {
  if (H <= 0 || H % 64 || H > 65536) { *why = "H must be a positive multiple of 64 (<= 65536)"; return false; }
  if (I <= 0 || I % 64 || I > 65536) { *why = "I must be a positive multiple of 64 (<= 65536)"; return false; }
  if (E < 1 || E > 512) { *why = "E must be in 1..512"; return false; }
  if (S < 0 || S > 64) { *why = "S must be in 0..64"; return false; }
  if (K < 1 || K > 16 || K > E) { *why = "K must be in 1..min(E,16)"; return false; }
  return true;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(int T, int H, int I, int E, int S, int K, bool bf16) {
  WsLayout L{};
  const size_t NB = (size_t)E + S, P = (size_t)T * (K + S);
  size_t off = 0;
  L.counts = off;  off += align256(NB * 4);
  L.offsets = off; off += align256((NB + 1) * 4);
  L.ptok = off;    off += align256(P * 4);
  L.pw = off;      off += align256(P * 4);
  L.ent = off;     off += align256(P * 4);
  L.max_items = max_decode_items(T, E, S, K);
  L.items = off;   off += align256((size_t)L.max_items * 4);
  L.items_dn = off; off += align256((size_t)L.max_items * 4);
  L.max_items_w = ffn_wide_from(T, H, I, E, S, K) ? max_wide_items(T, E, S, K) : 0;
  L.items_w = off;  off += align256((size_t)L.max_items_w * 4);
  L.items_dnw = off; off += align256((size_t)L.max_items_w * 4);
  L.wblk = off;    off += L.max_items_w ? align256(NB * 4) : 0;
  L.n_items = off; off += 256;  // [4]
  L.ccnt = off;    off += align256((size_t)group_chunks(T, K) * E * 4);
  L.hhi = off;     off += align256(P * (size_t)I * 2);
  L.hlo = off;     off += align256(P * (size_t)I * 2);
  L.hpan_size = L.max_items_w ? hpan_bytes(T, I, E, S, K) : 0;
  L.hpan = off;    off += align256(L.hpan_size);
  L.y = off;       off += align256(P * (size_t)H * 4 * dn_splits(T, H, I, E, S, K));
  L.xh = off;      off += bf16 ? align256((size_t)T * H * 2) : 0;
  L.xsc = off;     off += bf16 ? align256((size_t)T * 4) : 0;
  L.total = off;
  return L;
}

}  // namespace mpb

namespace {

// FFN view of a call: workspace regions of layout L inside ws, tc token chunks
// per gate_up item.
mpb::FfnParams ffn_params(const mpb::WsLayout& L, char* ws, const void* X_dev, int x_dtype, int T,
                          const int32_t* topk_idx_dev, const float* topk_w_dev, const uint32_t* const* planes_dev,
                          const uint16_t* const* luts_dev, const int32_t* q_dev, float* out_dev, int tc) {
  mpb::FfnParams p{};
  p.xh = x_dtype == MPB_BF16 ? (const uint16_t*)(ws + L.xh) : (const uint16_t*)X_dev;
  p.xsc = x_dtype == MPB_BF16 ? (const int32_t*)(ws + L.xsc) : nullptr;
  p.T = T; p.H = g.H; p.I = g.I; p.E = g.E; p.S = g.S; p.K = g.K; p.NB = g.E + g.S;
  p.topk_idx = topk_idx_dev; p.topk_w = topk_w_dev;
  p.planes = planes_dev; p.luts = luts_dev; p.q = q_dev;
  p.counts = (int32_t*)(ws + L.counts);
  p.offsets = (int32_t*)(ws + L.offsets);
  p.ptok = (int32_t*)(ws + L.ptok);
  p.pw = (float*)(ws + L.pw);
  p.ent = (int32_t*)(ws + L.ent);
  p.items = (int32_t*)(ws + L.items);
  p.items_dn = (int32_t*)(ws + L.items_dn);
  p.n_items = (int32_t*)(ws + L.n_items);
  p.max_items = L.max_items;
  p.tpi = mpb::kChunkTokens * tc;
  p.tpi_dn = mpb::kChunkTokens;
  // no wide items unless the caller enables them (ffn_impl)
  p.items_w = (int32_t*)(ws + L.items_w);
  p.items_dnw = (int32_t*)(ws + L.items_dnw);
  p.max_items_w = L.max_items_w;
  p.wide_from = 0;
  p.tpi_w = mpb::kWideTokGu;
  p.tpi_dnw = mpb::kWideTokDn;
  p.hhi = (uint16_t*)(ws + L.hhi);
  p.hlo = (uint16_t*)(ws + L.hlo);
  p.wblk = (int32_t*)(ws + L.wblk);
  p.hpan = (uint16_t*)(ws + L.hpan);
  p.y = (float*)(ws + L.y);
  p.out = out_dev;
  p.dn_split = 1;
  p.dn_hcs = (g.I / 64 + 1) & ~1;
  return p;
}

int qmax_all() {
  int m = 3;
  for (int v : g.q) m = std::max(m, v);
  return m;
}

// FFN launches read q_i on the stream set_committed_bits writes it on, so the
// two are ordered, and page offloads wait for them through lower_ev. A stream
// under graph capture is accepted too: its kernels run when the graph is
// replayed, and ordering replays against commits is the caller's part.
bool stream_ok(hipStream_t s) {
  if (s == g.stream) return true;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(s, &st) == hipSuccess && st == hipStreamCaptureStatusActive;
}

}  // namespace

extern "C" {

const char* mpb_last_error(void) { return g_err.c_str(); }

int mpb_init(const mpb_layer_desc* d, int32_t* q_dev, const int32_t* q_init_host, void* stream) try {
  if (!d || !q_dev || !q_init_host) return fail(MPB_E_ARG, "mpb_init: null pointer");
  const char* why = "";
  if (!mpb::geometry_ok(d->H, d->I, d->E, d->S, d->K, &why))
    return fail(MPB_E_SHAPE, std::string("mpb_init: ") + why);
  const int nb = 2 * (d->E + d->S);
  for (int i = 0; i < nb; ++i)
    if (q_init_host[i] < 3 || q_init_host[i] > 8)
      return fail(MPB_E_RANGE, "mpb_init: initial q[" + std::to_string(i) + "] outside 3..8");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(q_dev, q_init_host, nb * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(e, "mpb_init: copy of q");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "mpb_init: stream sync");
  void* scr = nullptr;
  const int rs = resolve_scratch(&scr);
  if (rs) return rs;
  g.init = true;
  g.H = d->H; g.I = d->I; g.E = d->E; g.S = d->S; g.K = d->K;
  g.q_dev = q_dev;
  g.q.assign(q_init_host, q_init_host + nb);
  g.resident.assign(nb, 8);
  for (const Xfer& x : g.xfer)
    if (x.ev) (void)hipEventDestroy(x.ev);
  g.xfer.assign(nb, Xfer{});
  for (hipEvent_t ev : g.lower_ev)
    if (ev) (void)hipEventDestroy(ev);
  g.lower_ev.assign(nb, nullptr);
  g.stream = s;
  return MPB_OK;
} catch (...) {
  return fail(MPB_E_HIP, "mpb_init: unexpected exception");
}

size_t mpb_plane_page_bytes(int N, int Kd) {
  if (N <= 0 || Kd <= 0) return 0;
  return (size_t)N * mpb::page_chunks(Kd) * 16;
}

int mpb_pack_block(const uint32_t* canon_dev, int N, int Kd, uint32_t* const* plane_pages_host,
                   void* stream) try {
  if (!canon_dev || !plane_pages_host) return fail(MPB_E_ARG, "mpb_pack_block: null pointer");
  for (int p = 0; p < 8; ++p)
    if (!plane_pages_host[p]) return fail(MPB_E_ARG, "mpb_pack_block: null page pointer");
  if (N <= 0 || N % 32 || Kd <= 0 || Kd % 64)
    return fail(MPB_E_SHAPE, "mpb_pack_block: need N % 32 == 0 and Kd % 64 == 0");
  hipError_t e = mpb::launch_pack(canon_dev, N, Kd, plane_pages_host, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mpb_pack_block");
  return MPB_OK;
} catch (...) {
  return fail(MPB_E_HIP, "mpb_pack_block: unexpected exception");
}

int64_t mpb_table_image_bytes(int kind, int N, int b) {
  if (kind != 0 && kind != 1) return fail(MPB_E_ARG, "mpb_table_image_bytes: kind must be 0 or 1");
  if (b < 3 || b > 8) return fail(MPB_E_RANGE, "mpb_table_image_bytes: b outside 3..8");
  if (N <= 0 || N % (kind == 0 ? 128 : 64) || N > 131072)
    return fail(MPB_E_SHAPE, "mpb_table_image_bytes: N must be a multiple of 128 (gate_up) or 64 (down)");
  return (int64_t)((N + 127) / 128) * (256 << b);
}

int mpb_pack_table(int kind, const uint16_t* lut_dev, int N, int b, uint16_t* image_dev, void* stream) try {
  const int64_t n = mpb_table_image_bytes(kind, N, b);
  if (n < 0) return (int)n;
  if (!lut_dev || !image_dev) return fail(MPB_E_ARG, "mpb_pack_table: null pointer");
  hipError_t e = mpb::launch_pack_table(lut_dev, kind, N, b, image_dev, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mpb_pack_table");
  return MPB_OK;
} catch (...) {
  return fail(MPB_E_HIP, "mpb_pack_table: unexpected exception");
}

int mpb_dequant_block(const uint32_t* const* pages_host, const uint16_t* lut_b_dev, int N, int Kd, int b,
                      uint16_t* out_f16_dev, void* stream) try {
  if (!pages_host || !lut_b_dev || !out_f16_dev) return fail(MPB_E_ARG, "mpb_dequant_block: null pointer");
  if (b < 3 || b > 8) return fail(MPB_E_RANGE, "mpb_dequant_block: b outside 3..8");
  for (int p = 0; p < b; ++p)
    if (!pages_host[p]) return fail(MPB_E_ARG, "mpb_dequant_block: null page pointer");
  if (N <= 0 || N % 32 || Kd <= 0 || Kd % 64)
    return fail(MPB_E_SHAPE, "mpb_dequant_block: need N % 32 == 0 and Kd % 64 == 0");
  hipError_t e = mpb::launch_dequant(pages_host, lut_b_dev, N, Kd, b, out_f16_dev, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mpb_dequant_block");
  return MPB_OK;
} catch (...) {
  return fail(MPB_E_HIP, "mpb_dequant_block: unexpected exception");
}

int mpb_dequant_block_image(const uint32_t* const* pages_host, const uint16_t* image_dev, int kind, int N, int Kd,
                            int b, uint16_t* out_f16_dev, void* stream) try {
  if (!pages_host || !image_dev || !out_f16_dev) return fail(MPB_E_ARG, "mpb_dequant_block_image: null pointer");
  if (kind != 0 && kind != 1) return fail(MPB_E_ARG, "mpb_dequant_block_image: kind must be 0 or 1");
  if (b < 3 || b > 8) return fail(MPB_E_RANGE, "mpb_dequant_block_image: b outside 3..8");
  for (int p = 0; p < b; ++p)
    if (!pages_host[p]) return fail(MPB_E_ARG, "mpb_dequant_block_image: null page pointer");
  if (N <= 0 || N % (kind == 0 ? 128 : 64) || Kd <= 0 || Kd % 64)
    return fail(MPB_E_SHAPE, "mpb_dequant_block_image: need N % 128 == 0 (kind 0) or N % 64 == 0 (kind 1), "
                             "and Kd % 64 == 0");
  hipError_t e = mpb::launch_dequant_image(pages_host, image_dev, kind, N, Kd, b, out_f16_dev, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mpb_dequant_block_image");
  return MPB_OK;
} catch (...) {
  return fail(MPB_E_HIP, "mpb_dequant_block_image: unexpected exception");
}

int moe_routing_mass(const int32_t* topk_idx_dev, const float* topk_w_dev, int T, int E, int K, double* mass_dev,
                     void* stream) try {
  if (T < 0 || T > (1 << 20)) return fail(MPB_E_SHAPE, "moe_routing_mass: T outside 0..2^20");
  if (E < 1 || E > 512) return fail(MPB_E_SHAPE, "moe_routing_mass: E must be in 1..512");
  if (K < 1 || K > 16 || K > E) return fail(MPB_E_SHAPE, "moe_routing_mass: K must be in 1..min(E,16)");
  if (!mass_dev || (T > 0 && (!topk_idx_dev || !topk_w_dev))) return fail(MPB_E_ARG, "moe_routing_mass: null pointer");
  hipError_t e = mpb::launch_routing_mass(topk_idx_dev, topk_w_dev, T, E, K, mass_dev, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_routing_mass");
  return MPB_OK;
} catch (...) {
  return fail(MPB_E_HIP, "moe_routing_mass: unexpected exception");
}

size_t moe_route_workspace_bytes(int T, int E) {
  if (T < 0 || E < 1 || E > 512) return 0;
  return mpb::route_workspace_bytes(T, E);
}

int moe_route(const void* X_dev, int x_dtype, const float* W_router_dev, const float* bias_dev, int T, int H,
              int E, int K, int32_t* topk_idx_dev, float* topk_w_dev, void* ws_dev, size_t ws_bytes,
              void* stream) try {
  if (x_dtype != MPB_F16 && x_dtype != MPB_BF16) return fail(MPB_E_ARG, "moe_route: bad x_dtype");
  if (T < 0) return fail(MPB_E_ARG, "moe_route: T < 0");
  if (T > (1 << 20)) return fail(MPB_E_SHAPE, "moe_route: T above 2^20");
  if (H <= 0 || H % 64 || H > 65536) return fail(MPB_E_SHAPE, "moe_route: H must be a multiple of 64 in 64..65536");
  if (E < 1 || E > 512) return fail(MPB_E_SHAPE, "moe_route: E must be in 1..512");
  if (K < 1 || K > 16 || K > E) return fail(MPB_E_SHAPE, "moe_route: K must be in 1..min(E,16)");
  if (T == 0) return MPB_OK;
  if (!X_dev || !W_router_dev || !topk_idx_dev || !topk_w_dev || !ws_dev)
    return fail(MPB_E_ARG, "moe_route: null pointer");
  const size_t need = mpb::route_workspace_bytes(T, E);
  if (ws_bytes < need)
    return fail(MPB_E_WS, "moe_route: workspace " + std::to_string(ws_bytes) + " < " + std::to_string(need));
  hipError_t e = mpb::launch_route((const uint16_t*)X_dev, x_dtype, W_router_dev, bias_dev, T, H, E, K,
                                   topk_idx_dev, topk_w_dev, (double*)ws_dev, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_route");
  return MPB_OK;
} catch (...) {
  return fail(MPB_E_HIP, "moe_route: unexpected exception");
}

size_t moe_ffn_workspace_bytes(int T) {
  if (!g.init || T < 0) return 0;
  // sized for bf16 activations (the larger case)
  return mpb::ws_layout(T, g.H, g.I, g.E, g.S, g.K, true).total;
}

}  // extern "C"

namespace {

// moe_ffn and moe_ffn_static: validation, workspace check and the launches.
// static_ws: the workspace is this device's scratch array (the size check then
// names its limit).
int ffn_impl(const char* name, const void* X_dev, int x_dtype, int T, const int32_t* topk_idx_dev,
             const float* topk_w_dev, const uint32_t* const* planes_dev, const uint16_t* const* luts_dev,
             const int32_t* q_dev, float* out_dev, void* ws_dev, size_t ws_bytes, void* stream, bool static_ws) {
  const std::string n(name);
  if (!g.init) return fail(MPB_E_UNINIT, n + ": no layer bound (mpb_init)");
  if (x_dtype != MPB_F16 && x_dtype != MPB_BF16) return fail(MPB_E_ARG, n + ": bad x_dtype");
  if (T < 0) return fail(MPB_E_ARG, n + ": T < 0");
  if (T == 0) return MPB_OK;
  if (T > (1 << 20)) return fail(MPB_E_SHAPE, n + ": T above 2^20");
  if (!X_dev || !topk_idx_dev || !topk_w_dev || !planes_dev || !luts_dev || !q_dev || !out_dev || !ws_dev)
    return fail(MPB_E_ARG, n + ": null pointer");
  if (q_dev != g.q_dev) return fail(MPB_E_ARG, n + ": q_dev is not the bound page table");
  if (!stream_ok((hipStream_t)stream))
    return fail(MPB_E_ARG, n + ": stream is neither the bound stream nor under graph capture");
  const mpb::WsLayout L = mpb::ws_layout(T, g.H, g.I, g.E, g.S, g.K, x_dtype == MPB_BF16);
  const long long ntile = std::max(g.I / 64, (g.H + 127) / 128);
  if (((long long)L.max_items + 7) / 8 * 8 * ntile * mpb::dn_splits(T, g.H, g.I, g.E, g.S, g.K) >= (1ll << 31) ||
      !mpb::rows_fit(L, T, g.H, g.I, g.K, g.S))
    return fail(MPB_E_SHAPE, n + ": T too large for this layer");
  if (ws_bytes < L.total) {
    if (static_ws)
      return fail(MPB_E_WS, n + ": " + std::to_string(T) + " tokens need " + std::to_string(L.total) +
                                " workspace bytes, above the static scratch limit of " + std::to_string(ws_bytes));
    return fail(MPB_E_WS, n + ": workspace " + std::to_string(ws_bytes) + " < " + std::to_string(L.total));
  }
  char* ws = (char*)ws_dev;
  // with the wide kernels taking the large groups, the rest are small: they
  // take 32-token items
  const int tc = mpb::ffn_wide_from(T, g.H, g.I, g.E, g.S, g.K) ? 1 : mpb::ffn_token_chunks(T, g.E, g.K);
  mpb::FfnParams p = ffn_params(L, ws, X_dev, x_dtype, T, topk_idx_dev, topk_w_dev, planes_dev, luts_dev, q_dev,
                                out_dev, tc);
  p.dn_split = mpb::dn_splits(T, g.H, g.I, g.E, g.S, g.K);
  p.dn_hcs = mpb::dn_range_hcs(g.I, p.dn_split);
  p.wide_from = mpb::ffn_wide_from(T, g.H, g.I, g.E, g.S, g.K);
  hipStream_t s = (hipStream_t)stream;
  mark(0, s);
  hipError_t e = hipSuccess;
  if (x_dtype == MPB_BF16) {
    e = mpb::launch_x_to_f16((const uint16_t*)X_dev, (uint16_t*)(ws + L.xh), (int32_t*)(ws + L.xsc), T, g.H, s);
    if (e != hipSuccess) return hip_fail(e, (n + ": activation conversion").c_str());
  }
  e = mpb::launch_permute(p, (int32_t*)(ws + L.ccnt), s);
  if (e != hipSuccess) return hip_fail(e, (n + ": permute").c_str());
  int qmax_gu = 3, qmax_dn = 3;
  for (int i = 0; i < g.nb(); i += 2) {
    qmax_gu = std::max(qmax_gu, g.q[i]);
    qmax_dn = std::max(qmax_dn, g.q[i + 1]);
  }
  // events 1 and 2 time the gate_up kernels themselves: their launches record
  // them (the wide launch, when there is one, records the start, the other
  // launch the end)
  hipEvent_t e1 = g_nev >= 5 ? g_ev[1] : nullptr, e2 = g_nev >= 5 ? g_ev[2] : nullptr;
  if (p.wide_from) {
    e = mpb::launch_wide(p, true, qmax_gu, s, e1, nullptr);
    if (e != hipSuccess) return hip_fail(e, (n + ": wide gate_up").c_str());
    e1 = nullptr;
  }
  e = mpb::launch_gate_up(p, qmax_gu, tc, s, e1, e2);
  if (e != hipSuccess) return hip_fail(e, (n + ": gate_up").c_str());
  // events 5 and 6 (optional) time the down kernels themselves
  hipEvent_t e5 = g_nev == 7 ? g_ev[5] : nullptr, e6 = g_nev == 7 ? g_ev[6] : nullptr;
  if (p.wide_from) {
    e = mpb::launch_wide(p, false, qmax_dn, s, e5, nullptr);
    if (e != hipSuccess) return hip_fail(e, (n + ": wide down").c_str());
    e5 = nullptr;
  }
  e = mpb::launch_down(p, qmax_dn, tc == 1, s, e5, e6);
  if (e != hipSuccess) return hip_fail(e, (n + ": down").c_str());
  mark(3, s);
  e = mpb::launch_combine(p, s);
  if (e != hipSuccess) return hip_fail(e, (n + ": combine").c_str());
  mark(4, s);
  return MPB_OK;
}

}  // namespace

extern "C" {

int moe_ffn(const void* X_dev, int x_dtype, int T, const int32_t* topk_idx_dev, const float* topk_w_dev,
            const uint32_t* const* planes_dev, const uint16_t* const* luts_dev, const int32_t* q_dev,
            float* out_dev, void* ws_dev, size_t ws_bytes, void* stream) try {
  return ffn_impl("moe_ffn", X_dev, x_dtype, T, topk_idx_dev, topk_w_dev, planes_dev, luts_dev, q_dev, out_dev,
                  ws_dev, ws_bytes, stream, false);
} catch (...) {
  return fail(MPB_E_HIP, "moe_ffn: unexpected exception");
}

int moe_ffn_static(const void* X_dev, int x_dtype, int T, const int32_t* topk_idx_dev, const float* topk_w_dev,
                   const uint32_t* const* planes_dev, const uint16_t* const* luts_dev, const int32_t* q_dev,
                   float* out_dev, void* stream) try {
  if (!g.init) return fail(MPB_E_UNINIT, "moe_ffn_static: no layer bound (mpb_init)");
  void* scr = nullptr;
  const int rs = resolve_scratch(&scr);
  if (rs) return rs;
  return ffn_impl("moe_ffn_static", X_dev, x_dtype, T, topk_idx_dev, topk_w_dev, planes_dev, luts_dev, q_dev,
                  out_dev, scr, kScratchBytes, stream, true);
} catch (...) {
  return fail(MPB_E_HIP, "moe_ffn_static: unexpected exception");
}

size_t moe_fused_counter_bytes(void) { return mpb::fused_counter_bytes(); }

size_t moe_fused_workspace_bytes(int T) {
  if (!g.init || T < 0) return 0;
  return mpb::fused_counter_bytes() + mpb::route_workspace_bytes(T, g.E) +
         mpb::ws_layout(T, g.H, g.I, g.E, g.S, g.K, true).total;
}

int moe_fused(const void* X_dev, int x_dtype, int T, const float* W_router_dev, const float* bias_dev,
              int32_t* topk_idx_dev, float* topk_w_dev, const uint32_t* const* planes_dev,
              const uint16_t* const* luts_dev, const int32_t* q_dev, float* out_dev, void* ws_dev, size_t ws_bytes,
              void* stream) try {
  if (!g.init) return fail(MPB_E_UNINIT, "moe_fused: no layer bound (mpb_init)");
  if (x_dtype != MPB_F16 && x_dtype != MPB_BF16) return fail(MPB_E_ARG, "moe_fused: bad x_dtype");
  if (T < 0) return fail(MPB_E_ARG, "moe_fused: T < 0");
  if (T == 0) return MPB_OK;
  if (T > (1 << 20)) return fail(MPB_E_SHAPE, "moe_fused: T above 2^20");
  if (!X_dev || !W_router_dev || !topk_idx_dev || !topk_w_dev || !planes_dev || !luts_dev || !q_dev || !out_dev ||
      !ws_dev)
    return fail(MPB_E_ARG, "moe_fused: null pointer");
  if ((uintptr_t)ws_dev % 256) return fail(MPB_E_ARG, "moe_fused: workspace not 256-byte aligned");
  if (q_dev != g.q_dev) return fail(MPB_E_ARG, "moe_fused: q_dev is not the bound page table");
  if (!stream_ok((hipStream_t)stream))
    return fail(MPB_E_ARG, "moe_fused: stream is neither the bound stream nor under graph capture");
  const mpb::WsLayout L = mpb::ws_layout(T, g.H, g.I, g.E, g.S, g.K, x_dtype == MPB_BF16);
  const long long ntile = std::max(g.I / 64, (g.H + 127) / 128);
  if ((long long)L.max_items * ntile * mpb::dn_splits(T, g.H, g.I, g.E, g.S, g.K) >= (1ll << 30) ||
      !mpb::rows_fit(L, T, g.H, g.I, g.K, g.S))
    return fail(MPB_E_SHAPE, "moe_fused: T too large for this layer");
  const size_t c_bytes = mpb::fused_counter_bytes(), r_bytes = mpb::route_workspace_bytes(T, g.E);
  const size_t need = c_bytes + r_bytes + L.total;
  if (ws_bytes < need)
    return fail(MPB_E_WS, "moe_fused: workspace " + std::to_string(ws_bytes) + " < " + std::to_string(need));
  char* ws = (char*)ws_dev;
  mpb::FusedLaunch F{};
  F.f = ffn_params(L, ws + c_bytes + r_bytes, X_dev, x_dtype, T, topk_idx_dev, topk_w_dev, planes_dev, luts_dev,
                   q_dev, out_dev, 1);
  F.f.dn_split = mpb::dn_splits(T, g.H, g.I, g.E, g.S, g.K);
  F.f.dn_hcs = mpb::dn_range_hcs(g.I, F.f.dn_split);
  F.x = (const uint16_t*)X_dev;
  F.xdt = x_dtype;
  F.W = W_router_dev;
  F.bias = bias_dev;
  F.logits = (double*)(ws + c_bytes);
  F.idx_out = topk_idx_dev;
  F.w_out = topk_w_dev;
  F.ctr = (uint32_t*)ws;
  F.qmax = qmax_all();
  const hipError_t e = mpb::launch_fused(F, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "moe_fused");
  return MPB_OK;
} catch (...) {
  return fail(MPB_E_HIP, "moe_fused: unexpected exception");
}

int set_committed_bits(int i, int b) try {
  if (!g.init) return fail(MPB_E_UNINIT, "set_committed_bits: no layer bound");
  if (i < 0 || i >= g.nb()) return fail(MPB_E_RANGE, "set_committed_bits: block index out of range");
  if (b < 3 || b > 8) return fail(MPB_E_RANGE, "set_committed_bits: bitwidth outside 3..8");
  const int rc = refresh_xfer(i);
  if (rc) return rc;
  if (b > g.resident[i])
    return fail(MPB_E_NOT_RESIDENT, "set_committed_bits: block " + std::to_string(i) + " has " +
                                        std::to_string(g.resident[i]) + " GPU-resident planes");
  hipError_t e = hipSuccess;
  if (b < g.q[i] && !g.lower_ev[i]) e = hipEventCreateWithFlags(&g.lower_ev[i], hipEventDisableTiming);
  if (e == hipSuccess) e = mpb::launch_set_q(g.q_dev, i, b, g.stream);
  if (e == hipSuccess && b < g.q[i]) e = hipEventRecord(g.lower_ev[i], g.stream);
  if (e != hipSuccess) return hip_fail(e, "set_committed_bits");
  g.q[i] = b;
  return MPB_OK;
} catch (...) {
  return fail(MPB_E_HIP, "set_committed_bits: unexpected exception");
}

int mpb_offload_pages(int i, int r, void* const* host_planes, const uint32_t* const* dev_planes,
                      void* const* host_tables, const uint16_t* const* dev_tables, void* copy_stream) try {
  if (!g.init) return fail(MPB_E_UNINIT, "mpb_offload_pages: no layer bound");
  if (i < 0 || i >= g.nb()) return fail(MPB_E_RANGE, "mpb_offload_pages: block index out of range");
  if (r < 3 || r > 8) return fail(MPB_E_RANGE, "mpb_offload_pages: page count outside 3..8");
  const int rc = refresh_xfer(i);
  if (rc) return rc;
  if (g.xfer[i].dir) return fail(MPB_E_BUSY, "mpb_offload_pages: a transfer of this block is in flight");
  if (g.q[i] > r) return fail(MPB_E_NOT_RESIDENT, "mpb_offload_pages: lower q_i to r before offloading");
  const int hi = g.resident[i];
  if (r >= hi) return MPB_OK;  // nothing above r is resident
  if (!page_ptrs_ok(r, hi, host_planes, (const void* const*)dev_planes, host_tables,
                    (const void* const*)dev_tables))
    return fail(MPB_E_ARG, "mpb_offload_pages: null pointer");
  hipStream_t cs = (hipStream_t)copy_stream;
  // a launch that may read a page above r was enqueued while q_i > r, i.e.
  // before the last lowering of q_i; the copies start after all of those, so
  // once they have completed no launch that reads these pages is left
  if (g.lower_ev[i]) {
    const hipError_t e = hipStreamWaitEvent(cs, g.lower_ev[i], 0);
    if (e != hipSuccess) return hip_fail(e, "mpb_offload_pages: ordering");
  }
  const int c = copy_pages(i, r, hi, host_planes, const_cast<uint32_t* const*>(dev_planes), host_tables,
                           const_cast<uint16_t* const*>(dev_tables), false, cs);
  if (c) return c;
  g.resident[i] = r;
  return MPB_OK;
} catch (...) {
  return fail(MPB_E_HIP, "mpb_offload_pages: unexpected exception");
}

int mpb_reload_pages(int i, int r, const void* const* host_planes, uint32_t* const* dev_planes,
                     const void* const* host_tables, uint16_t* const* dev_tables, void* copy_stream) try {
  if (!g.init) return fail(MPB_E_UNINIT, "mpb_reload_pages: no layer bound");
  if (i < 0 || i >= g.nb()) return fail(MPB_E_RANGE, "mpb_reload_pages: block index out of range");
  if (r < 3 || r > 8) return fail(MPB_E_RANGE, "mpb_reload_pages: page count outside 3..8");
  const int rc = refresh_xfer(i);
  if (rc) return rc;
  if (g.xfer[i].dir) return fail(MPB_E_BUSY, "mpb_reload_pages: a transfer of this block is in flight");
  const int lo = g.resident[i];
  if (r <= lo) return MPB_OK;  // already resident
  if (!page_ptrs_ok(lo, r, host_planes, (const void* const*)dev_planes, host_tables,
                    (const void* const*)dev_tables))
    return fail(MPB_E_ARG, "mpb_reload_pages: null pointer");
  return copy_pages(i, lo, r, const_cast<void* const*>(host_planes), dev_planes,
                    const_cast<void* const*>(host_tables), dev_tables, true, (hipStream_t)copy_stream);
} catch (...) {
  return fail(MPB_E_HIP, "mpb_reload_pages: unexpected exception");
}

int mpb_page_state(int i, int p) {
  if (!g.init) return fail(MPB_E_UNINIT, "mpb_page_state: no layer bound");
  if (i < 0 || i >= g.nb() || p < 0 || p > 7) return fail(MPB_E_RANGE, "mpb_page_state: index out of range");
  const int rc = refresh_xfer(i);
  if (rc) return rc;
  if (p < g.resident[i]) return MPB_PAGE_GPU;
  const Xfer& x = g.xfer[i];
  if (x.dir && p >= x.lo && p < x.hi) return MPB_PAGE_IN_TRANSFER;
  return MPB_PAGE_CPU;
}

int mpb_get_resident_planes(int i) {
  if (!g.init) return fail(MPB_E_UNINIT, "mpb_get_resident_planes: no layer bound");
  if (i < 0 || i >= g.nb()) return fail(MPB_E_RANGE, "mpb_get_resident_planes: block index out of range");
  const int rc = refresh_xfer(i);
  return rc ? rc : g.resident[i];
}

int mpb_set_kernel_events(void* const* events_host, int n) {
  if (n == 0) { g_nev = 0; return MPB_OK; }
  if ((n != 5 && n != 7) || !events_host) return fail(MPB_E_ARG, "mpb_set_kernel_events: need 5, 7 or 0 events");
  for (int k = 0; k < n; ++k) {
    if (!events_host[k]) return fail(MPB_E_ARG, "mpb_set_kernel_events: null event");
    g_ev[k] = (hipEvent_t)events_host[k];
  }
  g_nev = n;
  return MPB_OK;
}

int64_t mpb_committed_bytes(const uint8_t* touched_host) {
  if (!g.init) return fail(MPB_E_UNINIT, "mpb_committed_bytes: no layer bound");
  int64_t tot = 0;
  for (int i = 0; i < g.nb(); ++i) {
    if (touched_host && !touched_host[i]) continue;
    int N, Kd;
    block_shape(i, &N, &Kd);
    tot += block_bytes(N, Kd, g.q[i]);
  }
  return tot;
}

int mpb_get_committed_bits(int i) {
  if (!g.init) return fail(MPB_E_UNINIT, "mpb_get_committed_bits: no layer bound");
  if (i < 0 || i >= g.nb()) return fail(MPB_E_RANGE, "mpb_get_committed_bits: block index out of range");
  return g.q[i];
}

int mpb_set_resident_planes(int i, int r) {
  if (!g.init) return fail(MPB_E_UNINIT, "mpb_set_resident_planes: no layer bound");
  if (i < 0 || i >= g.nb()) return fail(MPB_E_RANGE, "mpb_set_resident_planes: block index out of range");
  if (r < 3 || r > 8) return fail(MPB_E_RANGE, "mpb_set_resident_planes: plane count outside 3..8");
  const int rc = refresh_xfer(i);
  if (rc) return rc;
  if (g.xfer[i].dir) return fail(MPB_E_BUSY, "mpb_set_resident_planes: a transfer of this block is in flight");
  if (r < g.q[i])
    return fail(MPB_E_NOT_RESIDENT, "mpb_set_resident_planes: lower q_i before offloading its planes");
  g.resident[i] = r;
  return MPB_OK;
}

}  // extern "C"
