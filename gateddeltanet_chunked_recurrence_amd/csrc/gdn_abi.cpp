// C ABI of the chunked gated delta rule library (declarations and contract in
// include/gdn.h). This layer validates every argument before any launch,
// reports failures through a status code and a thread-local message, and
// forwards to the HIP launchers. It allocates nothing and never synchronizes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/gdn.h"
#include "gdn_images.h"
#include "gdn_launch.h"

// Sticky device error flags (gdn::kErr* bits): kernels set them instead of
// failing silently, gdn_device_errors() reads and clears them. One copy per
// device (a file-scope device variable exists once on every GPU the library
// runs on).
__device__ __align__(256) uint32_t gdn_err_flags[64];

// Forward scratch of gdn_chunk_fwd_noalloc: a file-scope device array, so
// that entry point calls no allocator. Every GPU the library runs on holds
// its own copy until the process ends. Host code never passes this name to a
// kernel (on the host it is only a stand-in for the symbol): it uses the
// per-device address from scratch_ptr().
static __device__ __align__(256) uint8_t scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

// Device address of gdn_err_flags on the current device, looked up once per
// device (the host name of a device variable is not its device address).
uint32_t* err_word() {
  static std::mutex mu;
  static uint32_t* ptrs[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(gdn_err_flags)) != hipSuccess) return nullptr;
    ptrs[dev] = static_cast<uint32_t*>(p);
  }
  return ptrs[dev];
}

// Device address of `scratch` on the current device: hipGetSymbolAddress
// once per device (with that device current), then the cached pointer.
void* scratch_ptr() {
  static std::mutex mu;
  static void* ptrs[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

gdn_status fail(gdn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round256(int64_t x) { return (x + 255) & ~int64_t(255); }

bool valid_fmt(int32_t f) { return f == GDN_QDQ_OFF || f == GDN_QDQ_E4M3 || f == GDN_QDQ_INT8; }

// Shape and policy checks shared by forward and backward.
gdn_status check_fwd_shape(const gdn_fwd_args* a) {
  if (!a) return fail(GDN_E_INVALID, "argument struct is NULL");
  const gdn_qdq_policy& p = a->policy;
  if (p.chunk_size != 64)
    return fail(GDN_E_UNSUPPORTED, "chunk_size %d: only 64 is supported", p.chunk_size);
  if (p.solve_degree != 0 && p.solve_degree != 1 && p.solve_degree != 3 && p.solve_degree != 7 &&
      p.solve_degree != 15 && p.solve_degree != 31 && p.solve_degree != 63)
    return fail(GDN_E_UNSUPPORTED,
                "solve_degree %d: 0 (exact) or a Neumann degree 1, 3, 7, 15, 31 or 63",
                p.solve_degree);
  if (!valid_fmt(p.state_fmt) || !valid_fmt(p.w_fmt))
    return fail(GDN_E_UNSUPPORTED, "unknown QDQ format (state %d, w %d): use 0 off, 1 E4M3, 2 INT8",
                p.state_fmt, p.w_fmt);
  if (p.read_fmt != GDN_QDQ_OFF && p.read_fmt != GDN_QDQ_E4M3)
    return fail(GDN_E_UNSUPPORTED, "read_fmt %d: the two-precision read copy is E4M3 (1) or off (0)",
                p.read_fmt);
  if (a->B < 0 || a->T < 0 || a->Hqk <= 0 || a->Hv <= 0)
    return fail(GDN_E_INVALID, "bad sizes B=%d T=%d Hqk=%d Hv=%d", a->B, a->T, a->Hqk, a->Hv);
  if (a->Hv % a->Hqk != 0)
    return fail(GDN_E_INVALID, "Hv (%d) must be a multiple of Hqk (%d)", a->Hv, a->Hqk);
  if (a->Hv > 65535) return fail(GDN_E_UNSUPPORTED, "Hv %d exceeds 65535", a->Hv);
  if (a->Dk != 64 && a->Dk != 128)
    return fail(GDN_E_UNSUPPORTED, "Dk %d: supported 64, 128", a->Dk);
  if (a->Dv != 64 && a->Dv != 128 && a->Dv != 256)
    return fail(GDN_E_UNSUPPORTED, "Dv %d: supported 64, 128, 256", a->Dv);
  if (a->io_dtype != GDN_BF16 && a->io_dtype != GDN_F32)
    return fail(GDN_E_INVALID, "io_dtype %d: use 0 bf16 or 1 f32", a->io_dtype);
  if (a->io_dtype == GDN_F32 && a->Dk != 64)
    return fail(GDN_E_UNSUPPORTED, "FP32 inputs are built for Dk = 64 only (got %d)", a->Dk);
  if (a->io_dtype == GDN_F32 && p.solve_degree != 0)
    return fail(GDN_E_UNSUPPORTED, "the Neumann solve is built for bf16 inputs only");
  if (p.read_fmt != GDN_QDQ_OFF) {
    if (p.state_fmt != GDN_QDQ_OFF)
      return fail(GDN_E_INVALID, "read_fmt: the two-precision read copy replaces the state "
                                 "quantizer (state_fmt must be 0)");
    if (a->Dk != 128 || a->io_dtype != GDN_BF16)
      return fail(GDN_E_UNSUPPORTED, "read_fmt: the two-precision profile is built for Dk = 128 "
                                     "and bf16 inputs (Dk %d)", a->Dk);
  }
  if (p.state_fmt != GDN_QDQ_OFF) {
    if (p.block_v != 16 && p.block_v != 32 && p.block_v != 64 && p.block_v != 128 &&
        p.block_v != 256)
      return fail(GDN_E_UNSUPPORTED, "block_v %d: supported 16, 32, 64, 128, 256", p.block_v);
    if (a->Dv % p.block_v != 0)
      return fail(GDN_E_INVALID, "block_v %d does not divide Dv %d", p.block_v, a->Dv);
    if (a->io_dtype == GDN_F32 && p.block_v > 64)
      return fail(GDN_E_UNSUPPORTED, "FP32 inputs are built for block_v up to 64 (got %d)",
                  p.block_v);
  }
  if (!std::isfinite(a->scale)) return fail(GDN_E_INVALID, "scale is not finite");
  if (a->prefix_len < 0) return fail(GDN_E_INVALID, "prefix_len %d < 0", a->prefix_len);
  if (a->cu_seqlens) {
    if (a->B != 1) return fail(GDN_E_INVALID, "cu_seqlens needs B == 1 (got %d)", a->B);
    if (a->num_seqs < 1) return fail(GDN_E_INVALID, "num_seqs %d < 1 with cu_seqlens", a->num_seqs);
  } else if (a->num_seqs != a->B) {
    return fail(GDN_E_INVALID, "num_seqs (%d) must equal B (%d) without cu_seqlens",
                a->num_seqs, a->B);
  }
  if (a->num_seqs > 65535) return fail(GDN_E_UNSUPPORTED, "num_seqs %d exceeds 65535", a->num_seqs);
  if ((ceil_div((int64_t)a->B * a->T, 64) + a->num_seqs) * a->Hv > INT32_MAX)
    return fail(GDN_E_UNSUPPORTED, "(chunks + sequences) * Hv exceeds 2^31");
  if ((int64_t)a->B * a->T > INT32_MAX / 2)
    return fail(GDN_E_UNSUPPORTED, "B*T = %lld tokens exceeds 2^30", (long long)a->B * a->T);
  return GDN_OK;
}

gdn_status check_fwd_ptrs(const gdn_fwd_args* a, bool need_out) {
  const bool any = (int64_t)a->B * a->T > 0;
  const struct { const void* p; const char* name; bool required; } ptrs[] = {
      {a->q, "q", any},        {a->k, "k", any},      {a->v, "v", any},
      {a->g, "g", any},        {a->beta, "beta", any}, {a->o, "o", need_out && any},
      {a->h0, "h0", false},    {a->ht, "ht", false},  {a->cu_seqlens, "cu_seqlens", false},
      {a->saved, "saved", false}};
  for (const auto& e : ptrs) {
    if (e.required && !e.p) return fail(GDN_E_INVALID, "%s is NULL", e.name);
    if (e.p && !aligned16(e.p)) return fail(GDN_E_INVALID, "%s is not 16-byte aligned", e.name);
  }
  return GDN_OK;
}

gdn_saved_layout_t layout_of(const gdn_fwd_args* a) {
  gdn_saved_layout_t L{};
  const int64_t tokens = (int64_t)a->B * a->T;
  L.num_slots = a->num_seqs + ceil_div(tokens, 64);
  const int64_t per_state = (int64_t)a->Hv * a->Dk * a->Dv;
  const bool sq = a->policy.state_fmt != GDN_QDQ_OFF, wq = a->policy.w_fmt != GDN_QDQ_OFF;
  int64_t off = 0;
  L.off_state = off;
  off = round256(off + L.num_slots * per_state * (sq ? 1 : 4));
  L.off_state_scale = off;
  off = round256(off + (sq ? L.num_slots * a->Hv * (a->Dv / a->policy.block_v) * 4 : 0));
  L.off_w = off;
  off = round256(off + (wq ? tokens * a->Hv * a->Dk : 0));
  L.off_w_scale = off;
  off = round256(off + (wq ? L.num_slots * a->Hv * 4 : 0));
  L.off_x = off;
  off = round256(off + (a->io_dtype == GDN_BF16 ? L.num_slots * a->Hv * 64 * 64 * 4 : 0));
  L.off_anchor = off;
  off = round256(off + (a->policy.read_fmt != GDN_QDQ_OFF ? L.num_slots * per_state * 4 : 0));
  L.off_meta = off;
  off = round256(off + 64);
  L.total_bytes = off;
  return L;
}

// Forward scratch (bf16 io), per chunk slot and value head, 256-byte aligned
// sections: the operand image block [W planes | K^T | P] (bf16), U and the W
// scale (FP32).
struct FwdWsLayout {
  int64_t img, u, wscale, flags, vplan, total;
};

template <int DK>
FwdWsLayout fwd_ws_layout_dk(const gdn_fwd_args* a, int64_t nch) {
  using I = gdn::Img<DK>;
  const int64_t img = a->policy.w_fmt == GDN_QDQ_OFF ? I::template img<2>() : I::template img<1>();
  FwdWsLayout w{};
  int64_t off = 0;
  w.img = off;     off += round256(nch * img * 2);
  w.u = off;       off += round256(nch * (int64_t)a->Dv * 64 * 4);
  w.wscale = off;  off += round256(nch * 4);
  // ready flags, two item counters and the CU admission table of the overlapped forward
  w.flags = off;   off += round256(nch * 4 + 8 + gdn::kAdmitWords * 4);
  // its item table for packed sequences: [items, head, -, -] then (n Hv + head, chunk) per item
  w.vplan = off;   off += a->cu_seqlens ? round256((2 * nch + 4) * 4) : 0;
  w.total = off;
  return w;
}

FwdWsLayout fwd_ws_layout(const gdn_fwd_args* a) {
  FwdWsLayout w{};
  if (a->io_dtype == GDN_F32 || (int64_t)a->B * a->T == 0) return w;
  const int64_t nch = layout_of(a).num_slots * a->Hv;
  return a->Dk == 128 ? fwd_ws_layout_dk<128>(a, nch) : fwd_ws_layout_dk<64>(a, nch);
}

gdn::FwdKernelArgs kernel_args(const gdn_fwd_args* a, void* saved) {
  gdn::FwdKernelArgs k{};
  k.q = a->q;
  k.k = a->k;
  k.v = a->v;
  k.g = a->g;
  k.beta = a->beta;
  k.h0 = a->h0;
  k.cu_seqlens = a->cu_seqlens;
  k.o = a->o;
  k.ht = a->ht;
  if (saved) {
    const gdn_saved_layout_t L = layout_of(a);
    char* base = static_cast<char*>(saved);
    if (a->policy.state_fmt != GDN_QDQ_OFF) {
      k.s_codes = reinterpret_cast<uint8_t*>(base + L.off_state);
      k.s_scale = reinterpret_cast<float*>(base + L.off_state_scale);
    } else {
      k.s_f32 = reinterpret_cast<float*>(base + L.off_state);
    }
    if (a->policy.w_fmt != GDN_QDQ_OFF) {
      k.w_codes = reinterpret_cast<uint8_t*>(base + L.off_w);
      k.w_scale = reinterpret_cast<float*>(base + L.off_w_scale);
    }
    if (a->io_dtype == GDN_BF16) k.s_X = reinterpret_cast<float*>(base + L.off_x);
    if (a->policy.read_fmt != GDN_QDQ_OFF) k.s_anchor = reinterpret_cast<float*>(base + L.off_anchor);
    k.s_meta = reinterpret_cast<uint32_t*>(base + L.off_meta);
  }
  k.err = err_word();
  k.T = a->T;
  k.prefix_len = a->prefix_len;
  k.Hqk = a->Hqk;
  k.Hv = a->Hv;
  k.Dv = a->Dv;
  k.block_v = a->policy.state_fmt != GDN_QDQ_OFF ? a->policy.block_v : 64;
  k.scale = a->scale;
  return k;
}

gdn::FwdConfig fwd_config(const gdn_fwd_args* a) {
  gdn::FwdConfig c{};
  c.Dk = a->Dk;
  c.Dv = a->Dv;
  c.N = a->num_seqs;
  c.Hv = a->Hv;
  c.state_fmt = a->policy.state_fmt;
  c.w_fmt = a->policy.w_fmt;
  c.f32_io = a->io_dtype == GDN_F32;
  c.block_v = a->policy.state_fmt != GDN_QDQ_OFF ? a->policy.block_v : 64;
  c.read_fmt = a->policy.read_fmt;
  return c;
}

// Backward workspace sections (each 256-byte aligned):
//   X      [num_slots, Hv, 64, 64] FP32   (I + L)^-1 of every chunk
//   W      [B*T, Hv, Dk] FP32             the W of the products (dequantized Wq, or W)
//   dstate [num_slots, Hv] x Dk x Dv FP32 gradient of the state at each chunk end
//   dvn    [num_slots, Hv] x 64 x Dv FP32 gradient of Vnew per chunk
//   dqk    [B*T, Hv, 2, Dk] FP32          dq, dk per value head before the group sum
// and for bf16 inputs the operands of the reverse recurrence:
//   bimg   [num_slots, Hv] x image block (K image, W^T planes, gates) bf16
//   a1     [num_slots, Hv] x 64 x Dv FP32 scale P^T dO
//   a2     [num_slots, Hv] x Dk x Dv FP32 scale (e^gamma Q)^T dO
struct BwdWsLayout {
  int64_t X, W, dstate, dvn, dqk, bimg, a1, a2, dX, flags, total;
};

BwdWsLayout bwd_ws_layout(const gdn_fwd_args* a) {
  const gdn_saved_layout_t L = layout_of(a);
  const int64_t tokens = (int64_t)a->B * a->T, S = L.num_slots, Hv = a->Hv;
  const bool bf = a->io_dtype == GDN_BF16;
  BwdWsLayout w{};
  int64_t off = 0;
  w.X = off;       off += round256(S * Hv * 64 * 64 * 4);
  w.W = off;       off += round256(tokens * Hv * a->Dk * 4);
  w.dstate = off;  off += round256(S * Hv * a->Dk * a->Dv * 4);
  w.dvn = off;     off += round256(S * Hv * 64 * a->Dv * 4);
  w.dqk = off;     off += round256(tokens * Hv * 2 * a->Dk * 4);
  w.bimg = off;    off += bf ? round256(S * Hv * gdn::bwd_img_elems(a->Dk, a->policy.w_fmt) * 2) : 0;
  w.a1 = off;      off += bf ? round256(S * Hv * 64 * a->Dv * 4) : 0;
  w.a2 = off;      off += bf ? round256(S * Hv * a->Dk * a->Dv * 4) : 0;
  w.dX = off;      off += a->policy.solve_degree > 0 ? round256(S * Hv * 64 * 64 * 4) : 0;
  w.flags = off;   off += bf ? round256(S * Hv * 4) : 0;   // ready flags of the overlapped backward
  w.total = off;
  return w;
}

// The policy and shape a saved buffer is written under.
gdn::SavedStamp stamp_of(const gdn_fwd_args* a) {
  gdn::SavedStamp st{};
  const gdn_qdq_policy& p = a->policy;
  const uint32_t fmts = (uint32_t)p.state_fmt | (uint32_t)p.w_fmt << 8 | (uint32_t)p.read_fmt << 16;
  const uint32_t w[] = {gdn::SavedStamp::kMagic, (uint32_t)GDN_ABI_VERSION, fmts,
                        (uint32_t)(p.state_fmt != GDN_QDQ_OFF ? p.block_v : 0),
                        (uint32_t)p.solve_degree, (uint32_t)a->B, (uint32_t)a->T,
                        (uint32_t)a->Hqk, (uint32_t)a->Hv, (uint32_t)a->Dk, (uint32_t)a->Dv,
                        (uint32_t)a->num_seqs, (uint32_t)a->io_dtype, (uint32_t)a->prefix_len};
  static_assert(sizeof(w) / sizeof(w[0]) <= 15, "stamp words");
  for (size_t i = 0; i < sizeof(w) / sizeof(w[0]); ++i) st.w[i] = w[i];
  uint32_t sb;
  std::memcpy(&sb, &a->scale, 4);
  st.w[15] = sb;
  return st;
}

gdn_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GDN_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_last_error(void) { return g_err; }

gdn_status gdn_device_errors(uint32_t* flags) {
  if (!flags) return fail(GDN_E_INVALID, "flags is NULL");
  uint32_t* w = err_word();
  if (!w) return fail(GDN_E_HIP, "device error word unavailable on the current device");
  gdn_status s = hip_status(hipDeviceSynchronize(), "gdn_device_errors synchronize");
  if (s != GDN_OK) return s;
  if ((s = hip_status(hipMemcpy(flags, w, 4, hipMemcpyDeviceToHost), "gdn_device_errors read")) !=
      GDN_OK)
    return s;
  const uint32_t zero = 0;
  return hip_status(hipMemcpy(w, &zero, 4, hipMemcpyHostToDevice), "gdn_device_errors clear");
}
int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

gdn_status gdn_saved_layout(const gdn_fwd_args* a, gdn_saved_layout_t* out) {
  gdn_status s = check_fwd_shape(a);
  if (s != GDN_OK) return s;
  if (!out) return fail(GDN_E_INVALID, "layout output is NULL");
  *out = layout_of(a);
  return GDN_OK;
}

size_t gdn_saved_bytes(const gdn_fwd_args* a) {
  if (check_fwd_shape(a) != GDN_OK) return 0;
  return (size_t)layout_of(a).total_bytes;
}

size_t gdn_fwd_workspace_bytes(const gdn_fwd_args* a) {
  if (check_fwd_shape(a) != GDN_OK) return 0;
  return (size_t)fwd_ws_layout(a).total;
}

}  // extern "C"

namespace {

// Stages of the forward: 1 = prep (every chunk and head), 2 = state recurrence.
// ------------------------------------------------------- overlapped forward
// With equal-length sequences, the state kernel's U workgroups (N Hv Dv / 64,
// or fewer with 128- or 256-wide scale tiles) leave CUs idle.
// The forward then runs one prep launch on the caller's stream, taking the
// (chunk, head) items in chunk-major order (chunk c of every sequence and
// head before chunk c + 1) from a shared counter: the first H items on every
// CU; past them, U of its workgroups end and the other R = CUs - U go on
// with the rest. The state kernel, on a second stream of the library's, is
// enqueued behind the flag reset only, so it finds every CU held by the prep
// and starts on the CUs the ending workgroups free, with no kernel boundary
// in between; it waits for each chunk's ready flags, which every prep item
// sets after draining its device-scope stores. H makes the remainder on R
// CUs take about as long as the state chain: with per-item prep time
// t_item ~ 3.7 t_chunk (the measured per-chunk state step), H = items -
// R chunks t_chunk / t_item, rounded to whole rounds of CUs items. The
// kernels, their arithmetic and its order are those of the serial schedule,
// so the results are the same bits.
struct OverlapPlan {
  bool two = false;   // two prep workgroups per CU, the rest on admitted CUs
  int items = -1;             // -1: run serially; packed sequences: the upper bound slots * Hv
  int head = 0, rest_blocks = 0;
  bool varlen = false;        // packed sequences: items and head are decided on the device
  float item_per_chunk = 0.f;
};

// Prep time per (chunk, head) item over the state kernel's time per chunk
// step beside it, measured on the B4 x T4096 x H16 x D128 workload: for the
// split kernel about 10.1 us against 2.7 us; for the general kernel (QDQ off,
// INT8 state with W off, 128-wide tiles) about 9.9 us against 5.5 to 5.8 us.
constexpr double kSplitItemPerChunk = 3.7;
constexpr double kGeneralItemPerChunk = 1.75;
// the same with two prep workgroups per CU (its CUs build items faster)
constexpr double kSplitItemPerChunk2 = 3.0;
constexpr double kGeneralItemPerChunk2 = 1.75;

// GDN_NO_OVERLAP in the environment (read once): every call runs its stages
// one after the other on the caller's stream. For profilers that serialize
// kernels, under which a kernel waiting for another one's ready flags would
// wait out its bound.
bool overlap_disabled() {
  static const bool off = std::getenv("GDN_NO_OVERLAP") != nullptr;
  return off;
}

// with both QDQ sites on, the state kernel widens the W codes itself, so the
// images carry them as bytes (the split state kernel, which takes them, spans
// 64 columns: scale tiles up to 64 wide)
int w_img_bytes_of(const gdn_fwd_args* a) {
  return (a->policy.state_fmt != GDN_QDQ_OFF && a->policy.w_fmt != GDN_QDQ_OFF &&
          a->policy.block_v <= 64) ? 1 : 0;
}

OverlapPlan overlap_plan(const gdn_fwd_args* a, int cus) {
  OverlapPlan op;
  if (overlap_disabled() || a->io_dtype != GDN_BF16 || a->policy.read_fmt != 0) return op;
  // packed sequences: the setup kernel's limits (1,024 sequences, 4,095
  // chunks in the longest, which the total bounds)
  if (a->cu_seqlens && (a->num_seqs > 1024 || (int64_t)a->B * a->T > 4095LL * 64)) return op;
  const int len = a->prefix_len > 0 ? std::min(a->T, a->prefix_len) : a->T;
  const int maxc = (len + 63) / 64;
  const int64_t nh = (int64_t)a->num_seqs * a->Hv;
  // state workgroups: 64 value columns each, or a whole 128- or 256-wide
  // scale tile in the general kernel; and the measured prep time per item
  // over the kernel's time per chunk step
  const bool split = w_img_bytes_of(a) != 0;
  const int cols = !split && a->policy.state_fmt != GDN_QDQ_OFF && a->policy.block_v > 64
                       ? a->policy.block_v : 64;
  const double item_per_chunk = split ? kSplitItemPerChunk : kGeneralItemPerChunk;
  const int64_t units = nh * (a->Dv / cols);
  const int64_t rest = cus - units;
  if (rest < 16) return op;
  if (a->cu_seqlens) {
    op.items = (int)(layout_of(a).num_slots * a->Hv);
    op.head = -1;
    op.rest_blocks = (int)rest;
    op.varlen = true;
    op.item_per_chunk = (float)item_per_chunk;
    return op;
  }
  if (maxc < 4) return op;
  const int64_t items = (int64_t)maxc * nh;
  // with two prep workgroups per CU (its CUs build items faster) where
  // there is a head; the rest then runs on whole CUs that the admission
  // table picks. Without a head one workgroup per CU builds every item
  // beside the chain, which measured faster than two.
  const bool two = gdn::prep_workgroups_per_cu(fwd_config(a), a->policy.solve_degree) == 2;
  const double r2 = split ? kSplitItemPerChunk2 : kGeneralItemPerChunk2;
  const double h2 = (double)items - (double)rest * maxc / r2;
  const double h = two && h2 > 0.0 ? h2 : (double)items - (double)rest * maxc / item_per_chunk;
  const int64_t head = h <= 0.0 ? 0 : (int64_t)(h / cus + 0.5) * cus;
  if (head >= items) return op;
  op.two = two && head > 0;
  op.items = (int)items;
  op.head = (int)head;
  op.rest_blocks = (int)rest;
  return op;
}

// Per-device second stream and fork / join events, created once. The record /
// wait sequence of one call runs under the device's lock, so host threads
// calling at once do not interleave on the shared events.
struct OverlapRes {
  hipStream_t s2 = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool ok = false, tried = false;
  std::mutex mu;
};
OverlapRes* overlap_res() {
  static OverlapRes res[64];
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  OverlapRes& r = res[dev];
  if (!r.tried) {
    r.tried = true;
    // both streams are on this device: the events order them without the
    // system-scope fences (for the host and other devices) of an event
    constexpr unsigned kFlags = hipEventDisableTiming | hipEventDisableSystemFence;
    r.ok = hipStreamCreateWithFlags(&r.s2, hipStreamNonBlocking) == hipSuccess &&
           hipEventCreateWithFlags(&r.fork, kFlags) == hipSuccess &&
           hipEventCreateWithFlags(&r.join, kFlags) == hipSuccess;
  }
  return r.ok ? &r : nullptr;
}

// Chunks of every sequence whose backward images are built on every CU before
// the reverse recurrence starts (it consumes the last chunk first). Beside
// the recurrence the image kernel runs one workgroup per CU and delivers a
// chunk of nh (sequence, head) items every nh t_img / CUs; the recurrence
// takes t_chunk per chunk. With t_img ~ kImgPerChunk t_chunk (measured on
// the forward+backward workload: about 21 us per item against 2.35 us per
// chunk step), the head covers the deficit, plus two chunks the first
// steps look ahead for.
int bwd_head_chunks(int maxc, int64_t nh) {
  constexpr double kImgPerChunk = 21.0 / 2.35;
  const double r = (double)nh * kImgPerChunk / gdn::device_cus();   // image / recurrence time per chunk
  const int deficit = r > 1.0 ? (int)std::ceil(maxc * (1.0 - 1.0 / r)) : 0;
  return std::min(maxc, deficit + 2);
}

hipError_t run_overlapped(const gdn_fwd_args* a, const gdn::FwdConfig& cfg, gdn::FwdKernelArgs k,
                          const OverlapPlan& op, char* flags_mem, char* vplan_mem, hipStream_t st) {
  OverlapRes* r = overlap_res();
  if (!r) return hipErrorNotReady;
  const int num_slots = (int)layout_of(a).num_slots;
  uint32_t* flags = reinterpret_cast<uint32_t*>(flags_mem);
  const int64_t nflags = (int64_t)num_slots * a->Hv;
  gdn::FwdKernelArgs prep = k;
  prep.chunk_major = 1;
  prep.flags = flags;
  prep.ticket = flags + nflags;
  prep.item_lo = 0;
  prep.item_hi = op.items;
  prep.item_split = op.head;
  prep.prep_rest = op.rest_blocks;
  // with two prep workgroups per CU the rest is built on the CUs that the
  // admission table picks, from a launch over every CU; with one, by the
  // first rest_blocks workgroups
  prep.admit = op.two ? flags + nflags + 2 : nullptr;
  prep.prep_blocks = op.head > 0 ? 0 : op.rest_blocks;   // every CU while there is a head
  gdn::FwdKernelArgs state = k;
  state.flags = flags;
  // The fork and join events are recorded by the launches themselves, at
  // their end, with no marker packet of their own.
  std::lock_guard<std::mutex> lk(r->mu);
  hipError_t e;
  if (op.varlen) {
    // flags and counters zeroed, and the item table and head split built
    // from the sequence lengths, by one kernel
    prep.vplan = reinterpret_cast<const int32_t*>(vplan_mem);
    prep.item_split = 0;
    prep.prep_blocks = 0;
    e = gdn::launch_varlen_setup(flags, nflags + 2 + gdn::kAdmitWords, reinterpret_cast<int32_t*>(vplan_mem),
                                 a->cu_seqlens, a->num_seqs, a->prefix_len, a->Hv,
                                 gdn::device_cus(), op.rest_blocks, op.item_per_chunk, st, r->fork);
  } else {
    e = gdn::launch_fill_u32(flags, nflags + 2 + gdn::kAdmitWords, 0u, st, r->fork);   // flags, counters, table
  }
  if (e != hipSuccess) return e;
  if ((e = gdn::launch_fwd_prep(cfg, prep, num_slots, st)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(r->s2, r->fork, 0)) != hipSuccess) return e;
  if ((e = gdn::launch_fwd_state(cfg, state, r->s2, r->join)) != hipSuccess) return e;
  return hipStreamWaitEvent(st, r->join, 0);
}

// noalloc: the workspace is the library's `scratch` array instead of the
// caller's (a->workspace and a->workspace_bytes are not read).
gdn_status chunk_fwd_stages(const gdn_fwd_args* a, void* stream, int stages, bool noalloc = false) {
  gdn_status s = check_fwd_shape(a);
  if (s != GDN_OK) return s;
  if ((s = check_fwd_ptrs(a, true)) != GDN_OK) return s;
  const FwdWsLayout W = fwd_ws_layout(a);
  void* wsp = a->workspace;
  if (noalloc) {
    if (W.total > (int64_t)GDN_NOALLOC_SCRATCH_BYTES)
      return fail(GDN_E_UNSUPPORTED,
                  "gdn_chunk_fwd_noalloc: this problem needs %lld bytes of forward scratch, above "
                  "the library's fixed %lld (use gdn_chunk_fwd with a workspace)",
                  (long long)W.total, (long long)GDN_NOALLOC_SCRATCH_BYTES);
    if ((int64_t)a->B * a->T == 0) return GDN_OK;
    wsp = W.total > 0 ? scratch_ptr() : nullptr;
    if (W.total > 0 && !wsp)
      return fail(GDN_E_HIP, "gdn_chunk_fwd_noalloc: no device address for the scratch array");
  } else {
    if (W.total > 0 && (!a->workspace || a->workspace_bytes < (size_t)W.total))
      return fail(GDN_E_WORKSPACE, "forward workspace of %zu bytes given, %lld needed",
                  a->workspace_bytes, (long long)W.total);
    if (a->workspace && !aligned16(a->workspace))
      return fail(GDN_E_INVALID, "workspace is not 16-byte aligned");
  }
  if ((int64_t)a->B * a->T == 0) return GDN_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  gdn::FwdKernelArgs k = kernel_args(a, a->saved);
  if (!k.err) return fail(GDN_E_HIP, "device error word unavailable on the current device");
  const gdn::FwdConfig cfg = fwd_config(a);
  if (k.s_meta && (stages & 2)) {
    s = hip_status(gdn::launch_write_stamp(k.s_meta, stamp_of(a), st), "gdn_chunk_fwd stamp");
    if (s != GDN_OK) return s;
  }
  if (a->io_dtype == GDN_F32)
    return (stages & 2) ? hip_status(gdn::launch_fwd_fused(cfg, k, st), "gdn_chunk_fwd launch")
                        : GDN_OK;
  char* ws = static_cast<char*>(wsp);
  k.ws_img = reinterpret_cast<__bf16*>(ws + W.img);
  k.ws_u = reinterpret_cast<float*>(ws + W.u);
  k.ws_wscale = reinterpret_cast<float*>(ws + W.wscale);
  k.w_img_bytes = w_img_bytes_of(a);
  k.solve_degree = a->policy.solve_degree;
  if (stages == 3 && !noalloc) {
    const OverlapPlan op = overlap_plan(a, gdn::device_cus());
    // (without the second stream the same kernels run one after the other)
    if (op.items >= 0 && overlap_res())
      return hip_status(run_overlapped(a, cfg, k, op, ws + W.flags, ws + W.vplan, st),
                        "gdn_chunk_fwd overlapped launch");
  }
  if (stages & 1) {
    const int num_slots = (int)layout_of(a).num_slots;
    s = hip_status(gdn::launch_fwd_prep(cfg, k, num_slots, st), "gdn_chunk_fwd prep launch");
    if (s != GDN_OK) return s;
  }
  if (stages & 2) return hip_status(gdn::launch_fwd_state(cfg, k, st), "gdn_chunk_fwd state launch");
  return GDN_OK;
}

// ------------------------------------------------------------------ decode
gdn_status check_decode(const gdn_decode_args* a) {
  if (!a) return fail(GDN_E_INVALID, "argument struct is NULL");
  if (a->B < 0 || a->T < 0 || a->Hqk <= 0 || a->Hv <= 0)
    return fail(GDN_E_INVALID, "bad sizes B=%d T=%d Hqk=%d Hv=%d", a->B, a->T, a->Hqk, a->Hv);
  if (a->Hv % a->Hqk != 0)
    return fail(GDN_E_INVALID, "Hv (%d) must be a multiple of Hqk (%d)", a->Hv, a->Hqk);
  if (a->Dk != 64 && a->Dk != 128) return fail(GDN_E_UNSUPPORTED, "Dk %d: supported 64, 128", a->Dk);
  if (a->Dv != 64 && a->Dv != 128 && a->Dv != 256)
    return fail(GDN_E_UNSUPPORTED, "Dv %d: supported 64, 128, 256", a->Dv);
  if (a->io_dtype != GDN_BF16 && a->io_dtype != GDN_F32)
    return fail(GDN_E_INVALID, "io_dtype %d: use 0 bf16 or 1 f32", a->io_dtype);
  if (!valid_fmt(a->state_fmt))
    return fail(GDN_E_UNSUPPORTED, "unknown state format %d: use 0 off, 1 E4M3, 2 INT8",
                a->state_fmt);
  if (a->state_fmt != GDN_QDQ_OFF) {
    if (a->block_v != 16 && a->block_v != 32 && a->block_v != 64 && a->block_v != 128 &&
        a->block_v != 256)
      return fail(GDN_E_UNSUPPORTED, "block_v %d: supported 16, 32, 64, 128, 256", a->block_v);
    if (a->Dv % a->block_v != 0)
      return fail(GDN_E_INVALID, "block_v %d does not divide Dv %d", a->block_v, a->Dv);
  }
  if (a->readout != GDN_READOUT_BEFORE_WRITE && a->readout != GDN_READOUT_AFTER_WRITE)
    return fail(GDN_E_INVALID, "readout %d: 0 before the write, 1 after it", a->readout);
  if (a->start < 0) return fail(GDN_E_INVALID, "start %d < 0", a->start);
  if (!std::isfinite(a->scale)) return fail(GDN_E_INVALID, "scale is not finite");
  if (a->cu_seqlens) {
    if (a->B != 1) return fail(GDN_E_INVALID, "cu_seqlens needs B == 1 (got %d)", a->B);
    if (a->num_seqs < 1) return fail(GDN_E_INVALID, "num_seqs %d < 1 with cu_seqlens", a->num_seqs);
  } else if (a->num_seqs != a->B) {
    return fail(GDN_E_INVALID, "num_seqs (%d) must equal B (%d) without cu_seqlens",
                a->num_seqs, a->B);
  }
  if ((int64_t)a->num_seqs * a->Hv > INT32_MAX)
    return fail(GDN_E_UNSUPPORTED, "num_seqs * Hv exceeds 2^31");
  if ((int64_t)a->B * a->T > INT32_MAX / 2)
    return fail(GDN_E_UNSUPPORTED, "B*T = %lld tokens exceeds 2^30", (long long)a->B * a->T);
  return GDN_OK;
}

gdn_status check_decode_ptrs(const gdn_decode_args* a, bool need_out) {
  const bool any = (int64_t)a->B * a->T > 0;
  const struct { const void* p; const char* name; bool required; } ptrs[] = {
      {a->q, "q", any},          {a->k, "k", any},      {a->v, "v", any},
      {a->g, "g", any},          {a->beta, "beta", any}, {a->o, "o", need_out && any},
      {a->h_in, "h_in", false},  {a->ht, "ht", false},  {a->cu_seqlens, "cu_seqlens", false},
      {a->saved, "saved", false}};
  for (const auto& e : ptrs) {
    if (e.required && !e.p) return fail(GDN_E_INVALID, "%s is NULL", e.name);
    if (e.p && !aligned16(e.p)) return fail(GDN_E_INVALID, "%s is not 16-byte aligned", e.name);
  }
  return GDN_OK;
}

// Saved written states: codes (or FP32 states), tile scales, the stamp.
struct DecodeLayout {
  int64_t slots, off_state, off_scale, off_meta, total;
};
DecodeLayout decode_layout(const gdn_decode_args* a) {
  DecodeLayout L{};
  L.slots = (int64_t)a->B * a->T + a->num_seqs;
  const int64_t per = (int64_t)a->Hv * a->Dk * a->Dv;
  const bool sq = a->state_fmt != GDN_QDQ_OFF;
  int64_t off = 0;
  L.off_state = off;
  off = round256(off + L.slots * per * (sq ? 1 : 4));
  L.off_scale = off;
  off = round256(off + (sq ? L.slots * a->Hv * (a->Dv / a->block_v) * 4 : 0));
  L.off_meta = off;
  L.total = round256(off + 64);
  return L;
}

gdn::SavedStamp decode_stamp(const gdn_decode_args* a) {
  gdn::SavedStamp st{};
  const uint32_t w[] = {0x44444E47u /* "GNDD" */, (uint32_t)GDN_ABI_VERSION,
                        (uint32_t)a->state_fmt,
                        (uint32_t)(a->state_fmt != GDN_QDQ_OFF ? a->block_v : 0),
                        (uint32_t)a->readout, (uint32_t)a->start, (uint32_t)a->B,
                        (uint32_t)a->T, (uint32_t)a->Hqk, (uint32_t)a->Hv, (uint32_t)a->Dk,
                        (uint32_t)a->Dv, (uint32_t)a->num_seqs, (uint32_t)a->io_dtype};
  static_assert(sizeof(w) / sizeof(w[0]) <= 15, "stamp words");
  for (size_t i = 0; i < sizeof(w) / sizeof(w[0]); ++i) st.w[i] = w[i];
  uint32_t sb;
  std::memcpy(&sb, &a->scale, 4);
  st.w[15] = sb;
  return st;
}

gdn::DecodeKernelArgs decode_kernel_args(const gdn_decode_args* a) {
  gdn::DecodeKernelArgs k{};
  k.q = a->q;
  k.k = a->k;
  k.v = a->v;
  k.g = a->g;
  k.beta = a->beta;
  k.h_in = a->h_in;
  k.cu_seqlens = a->cu_seqlens;
  k.o = a->o;
  k.ht = a->ht;
  if (a->saved) {
    const DecodeLayout L = decode_layout(a);
    char* base = static_cast<char*>(a->saved);
    if (a->state_fmt != GDN_QDQ_OFF) {
      k.s_codes = reinterpret_cast<uint8_t*>(base + L.off_state);
      k.s_scale = reinterpret_cast<float*>(base + L.off_scale);
    } else {
      k.s_f32 = reinterpret_cast<float*>(base + L.off_state);
    }
  }
  k.T = a->T;
  k.start = a->start;
  k.Hqk = a->Hqk;
  k.Hv = a->Hv;
  k.Dv = a->Dv;
  k.block_v = a->state_fmt != GDN_QDQ_OFF ? a->block_v : 64;
  k.readout = a->readout;
  k.num_seqs = a->num_seqs;
  k.scale = a->scale;
  k.total_tokens = (int32_t)((int64_t)a->B * a->T);
  return k;
}

gdn::DecodeConfig decode_config(const gdn_decode_args* a) {
  gdn::DecodeConfig c{};
  c.Dk = a->Dk;
  c.Dv = a->Dv;
  c.N = a->num_seqs;
  c.Hv = a->Hv;
  c.Hqk = a->Hqk;
  c.state_fmt = a->state_fmt;
  c.f32_io = a->io_dtype == GDN_F32;
  return c;
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_fwd(const gdn_fwd_args* a, void* stream) { return chunk_fwd_stages(a, stream, 3); }
gdn_status gdn_chunk_fwd_noalloc(const gdn_fwd_args* a, void* stream) {
  return chunk_fwd_stages(a, stream, 3, true);
}
gdn_status gdn_chunk_fwd_prep(const gdn_fwd_args* a, void* stream) {
  return chunk_fwd_stages(a, stream, 1);
}
gdn_status gdn_chunk_fwd_state(const gdn_fwd_args* a, void* stream) {
  return chunk_fwd_stages(a, stream, 2);
}

gdn_status gdn_fwd_schedule(const gdn_fwd_args* a, int32_t cus, int32_t* out) {
  gdn_status s = check_fwd_shape(a);
  if (s != GDN_OK) return s;
  if (!out) return fail(GDN_E_INVALID, "out is NULL");
  if (cus < 0) return fail(GDN_E_INVALID, "cus %d < 0", cus);
  const OverlapPlan op = overlap_plan(a, cus > 0 ? cus : gdn::device_cus());
  out[0] = op.items >= 0 ? 1 : 0;
  out[1] = op.varlen ? -1 : (op.items >= 0 ? op.items : 0);
  out[2] = op.head;
  out[3] = op.rest_blocks;
  return GDN_OK;
}

size_t gdn_bwd_workspace_bytes(const gdn_bwd_args* a) {
  if (!a || check_fwd_shape(&a->fwd) != GDN_OK) return 0;
  return (size_t)bwd_ws_layout(&a->fwd).total;
}

gdn_status gdn_chunk_bwd(const gdn_bwd_args* a, void* stream) {
  if (!a) return fail(GDN_E_INVALID, "argument struct is NULL");
  gdn_status s = check_fwd_shape(&a->fwd);
  if (s != GDN_OK) return s;
  if ((s = check_fwd_ptrs(&a->fwd, false)) != GDN_OK) return s;
  const bool any = (int64_t)a->fwd.B * a->fwd.T > 0;
  if (a->grad_dtype != GDN_F32 && a->grad_dtype != a->fwd.io_dtype)
    return fail(GDN_E_INVALID, "grad_dtype must be FP32 or the io dtype");
  const struct { const void* p; const char* name; bool required; } ptrs[] = {
      {a->fwd.saved, "saved", any}, {a->do_, "do", any},  {a->dq, "dq", any},
      {a->dk, "dk", any},           {a->dv, "dv", any},   {a->dg, "dg", any},
      {a->dbeta, "dbeta", any},     {a->dht, "dht", false}, {a->dh0, "dh0", false},
      {a->workspace, "workspace", false}};
  for (const auto& e : ptrs) {
    if (e.required && !e.p) return fail(GDN_E_INVALID, "%s is NULL", e.name);
    if (e.p && !aligned16(e.p)) return fail(GDN_E_INVALID, "%s is not 16-byte aligned", e.name);
  }
  const size_t need = gdn_bwd_workspace_bytes(a);
  if (any && (!a->workspace || a->workspace_bytes < need))
    return fail(GDN_E_WORKSPACE, "workspace of %zu bytes given, %zu needed", a->workspace_bytes, need);
  if (!any) return GDN_OK;
  const gdn_saved_layout_t L = layout_of(&a->fwd);
  const int64_t tokens = (int64_t)a->fwd.B * a->fwd.T;
  gdn::BwdKernelArgs k{};
  k.f = kernel_args(&a->fwd, a->fwd.saved);
  k.dout = a->do_;
  k.dht = a->dht;
  k.dq = a->dq;
  k.dk = a->dk;
  k.dv = a->dv;
  k.dg = a->dg;
  k.dbeta = a->dbeta;
  k.dh0 = a->dh0;
  char* ws = static_cast<char*>(a->workspace);
  const BwdWsLayout W = bwd_ws_layout(&a->fwd);
  // bf16 inputs with W QDQ: X comes from the forward (saved); otherwise the
  // backward's first kernel solves again into the workspace
  // (with the approximate inverse the saved X is the polynomial, which no
  // exact solve may replace)
  k.ws_X = (k.f.s_X && (a->fwd.policy.w_fmt != GDN_QDQ_OFF || a->fwd.policy.solve_degree > 0))
               ? k.f.s_X
               : reinterpret_cast<float*>(ws + W.X);
  k.ws_dX = reinterpret_cast<float*>(ws + W.dX);
  k.f.solve_degree = a->fwd.policy.solve_degree;
  k.ws_W = reinterpret_cast<float*>(ws + W.W);
  k.ws_dstate = reinterpret_cast<float*>(ws + W.dstate);
  k.ws_dvn = reinterpret_cast<float*>(ws + W.dvn);
  k.ws_dqk = reinterpret_cast<float*>(ws + W.dqk);
  k.ws_bimg = reinterpret_cast<__bf16*>(ws + W.bimg);
  k.ws_a1 = reinterpret_cast<float*>(ws + W.a1);
  k.ws_a2 = reinterpret_cast<float*>(ws + W.a2);
  k.grad_f32 = a->grad_dtype == GDN_F32;
  k.total_tokens = (int32_t)tokens;
  k.num_slots = (int32_t)L.num_slots;
  gdn::BwdConfig c{};
  c.Dk = a->fwd.Dk;
  c.Dv = a->fwd.Dv;
  c.N = a->fwd.num_seqs;
  c.Hv = a->fwd.Hv;
  c.Hqk = a->fwd.Hqk;
  c.state_fmt = a->fwd.policy.state_fmt;
  c.w_fmt = a->fwd.policy.w_fmt;
  c.f32_io = a->fwd.io_dtype == GDN_F32;
  if (!k.f.err) return fail(GDN_E_HIP, "device error word unavailable on the current device");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  // Overlapped backward (equal-length bf16 sequences, where the image and the
  // state kernel fit on one CU together): the image kernel runs beside the
  // reverse recurrence on the library's second stream, in the chunk order the
  // recurrence consumes (its ready flags in the workspace), instead of before
  // it. Same kernels and arithmetic, so the same bits.
  {
    const int len = a->fwd.prefix_len > 0 ? std::min(a->fwd.T, a->fwd.prefix_len) : a->fwd.T;
    const int maxc = (len + 63) / 64;
    OverlapRes* r = nullptr;
    if (!overlap_disabled() && !c.f32_io && !a->fwd.cu_seqlens && maxc >= 4 &&
        gdn::bwd_overlap_fits(c) && (r = overlap_res())) {
      k.flags = reinterpret_cast<uint32_t*>(ws + W.flags);
      k.rev_maxc = maxc;
      k.rev_done = bwd_head_chunks(maxc, (int64_t)a->fwd.num_seqs * a->fwd.Hv);
      const gdn::BwdOverlap ov{r->s2, r->fork, r->join};
      std::lock_guard<std::mutex> lk(r->mu);
      s = hip_status(gdn::launch_bwd(c, k, st, &ov), "gdn_chunk_bwd overlapped launch");
    } else {
      s = hip_status(gdn::launch_bwd(c, k, st), "gdn_chunk_bwd launch");
    }
  }
  if (s != GDN_OK) return s;
  if (a->fwd.policy.read_fmt != GDN_QDQ_OFF) {
    s = hip_status(gdn::launch_bwd_read_anchor(c, k, st), "gdn_chunk_bwd anchor term");
    if (s != GDN_OK) return s;
  }
  // the saved buffer must come from a forward with this policy and shape
  const int64_t n_dqk = tokens * a->fwd.Hqk * a->fwd.Dk, n_dv = tokens * a->fwd.Hv * a->fwd.Dv;
  const int64_t n_h0 = (int64_t)a->fwd.num_seqs * a->fwd.Hv * a->fwd.Dk * a->fwd.Dv;
  return hip_status(gdn::launch_check_stamp(k, stamp_of(&a->fwd), n_dqk, n_dv, tokens * a->fwd.Hv,
                                            n_h0, st),
                    "gdn_chunk_bwd stamp check");
}

size_t gdn_decode_saved_bytes(const gdn_decode_args* a) {
  if (check_decode(a) != GDN_OK) return 0;
  return (size_t)decode_layout(a).total;
}

gdn_status gdn_decode_fwd(const gdn_decode_args* a, void* stream) {
  gdn_status s = check_decode(a);
  if (s != GDN_OK) return s;
  if ((s = check_decode_ptrs(a, true)) != GDN_OK) return s;
  if (a->num_seqs == 0 || (int64_t)a->B * a->T + a->num_seqs == 0) return GDN_OK;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const gdn::DecodeKernelArgs k = decode_kernel_args(a);
  if (a->saved) {
    s = hip_status(gdn::launch_write_stamp(reinterpret_cast<uint32_t*>(
                                               static_cast<char*>(a->saved) + decode_layout(a).off_meta),
                                           decode_stamp(a), st),
                   "gdn_decode_fwd stamp");
    if (s != GDN_OK) return s;
  }
  return hip_status(gdn::launch_decode_fwd(decode_config(a), k, st), "gdn_decode_fwd launch");
}

size_t gdn_decode_bwd_workspace_bytes(const gdn_decode_bwd_args* a) {
  if (!a || check_decode(&a->fwd) != GDN_OK) return 0;
  // partial dq, dk, dg, dbeta per (token, value head, group of slabs)
  const int ng = a->fwd.Dv / 64 / gdn::decode_slabs_per_group(a->fwd.state_fmt, a->fwd.block_v);
  if (a->fwd.Hv == a->fwd.Hqk && ng == 1) return 0;
  return (size_t)round256((int64_t)a->fwd.B * a->fwd.T * a->fwd.Hv * ng * (2 * a->fwd.Dk + 4) * 4);
}

gdn_status gdn_decode_bwd(const gdn_decode_bwd_args* a, void* stream) {
  if (!a) return fail(GDN_E_INVALID, "argument struct is NULL");
  gdn_status s = check_decode(&a->fwd);
  if (s != GDN_OK) return s;
  if ((s = check_decode_ptrs(&a->fwd, false)) != GDN_OK) return s;
  const int64_t tokens = (int64_t)a->fwd.B * a->fwd.T;
  if (a->grad_dtype != GDN_F32 && a->grad_dtype != a->fwd.io_dtype)
    return fail(GDN_E_INVALID, "grad_dtype must be FP32 or the io dtype");
  const bool any = tokens > 0;
  const struct { const void* p; const char* name; bool required; } ptrs[] = {
      {a->fwd.saved, "saved", true}, {a->do_, "do", any},    {a->dq, "dq", any},
      {a->dk, "dk", any},            {a->dv, "dv", any},     {a->dg, "dg", any},
      {a->dbeta, "dbeta", any},      {a->dht, "dht", false}, {a->dh_in, "dh_in", false},
      {a->workspace, "workspace", false}};
  for (const auto& e : ptrs) {
    if (e.required && !e.p) return fail(GDN_E_INVALID, "%s is NULL", e.name);
    if (e.p && !aligned16(e.p)) return fail(GDN_E_INVALID, "%s is not 16-byte aligned", e.name);
  }
  const size_t need = gdn_decode_bwd_workspace_bytes(a);
  if (need && (!a->workspace || a->workspace_bytes < need))
    return fail(GDN_E_WORKSPACE, "workspace of %zu bytes given, %zu needed", a->workspace_bytes, need);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  gdn::DecodeKernelArgs k = decode_kernel_args(&a->fwd);
  k.dout = a->do_;
  k.dht = a->dht;
  k.dq = a->dq;
  k.dk = a->dk;
  k.dv = a->dv;
  k.dg = a->dg;
  k.dbeta = a->dbeta;
  k.dh_in = a->dh_in;
  k.ws_dqk = need ? static_cast<float*>(a->workspace) : nullptr;
  k.grad_f32 = a->grad_dtype == GDN_F32;
  uint32_t* err = err_word();
  if (!err) return fail(GDN_E_HIP, "device error word unavailable on the current device");
  s = hip_status(gdn::launch_decode_bwd(decode_config(&a->fwd), k, st), "gdn_decode_bwd launch");
  if (s != GDN_OK) return s;
  // the saved buffer must come from a decode forward with this policy and shape
  gdn::BwdKernelArgs c{};
  c.f.s_meta = reinterpret_cast<uint32_t*>(static_cast<char*>(a->fwd.saved) +
                                           decode_layout(&a->fwd).off_meta);
  c.f.err = err;
  c.dq = a->dq;
  c.dk = a->dk;
  c.dv = a->dv;
  c.dg = a->dg;
  c.dbeta = a->dbeta;
  c.dh0 = a->dh_in;
  c.grad_f32 = k.grad_f32;
  const int64_t n_h = (int64_t)a->fwd.num_seqs * a->fwd.Hv * a->fwd.Dk * a->fwd.Dv;
  return hip_status(gdn::launch_check_stamp(c, decode_stamp(&a->fwd), tokens * a->fwd.Hqk * a->fwd.Dk,
                                            tokens * a->fwd.Hv * a->fwd.Dv, tokens * a->fwd.Hv, n_h,
                                            st),
                    "gdn_decode_bwd stamp check");
}

gdn_status gdn_qdq_state(const float* x, float* y, float* scales, uint8_t* codes,
                         int64_t n_states, int32_t Dk, int32_t Dv, int32_t block_v,
                         int32_t fmt, void* stream) {
  if (fmt != GDN_QDQ_E4M3 && fmt != GDN_QDQ_INT8)
    return fail(GDN_E_UNSUPPORTED, "gdn_qdq_state format %d: use 1 E4M3 or 2 INT8", fmt);
  if (n_states < 0 || Dk < 1 || Dk > 1024 || Dv < 1)
    return fail(GDN_E_INVALID, "bad sizes n_states=%lld Dk=%d Dv=%d", (long long)n_states, Dk, Dv);
  if (block_v != 16 && block_v != 32 && block_v != 64 && block_v != 128 && block_v != 256)
    return fail(GDN_E_UNSUPPORTED, "block_v %d: supported 16, 32, 64, 128, 256", block_v);
  if (Dv % block_v != 0) return fail(GDN_E_INVALID, "block_v %d does not divide Dv %d", block_v, Dv);
  if (n_states * (Dv / block_v) > INT32_MAX)
    return fail(GDN_E_UNSUPPORTED, "too many tiles");
  if (n_states == 0) return GDN_OK;
  if (!x || !y) return fail(GDN_E_INVALID, "x or y is NULL");
  const void* ps[] = {x, y, scales, codes};
  for (const void* p : ps)
    if (p && !aligned16(p)) return fail(GDN_E_INVALID, "pointer is not 16-byte aligned");
  return hip_status(gdn::launch_qdq_state(x, y, scales, codes, n_states, Dk, Dv, block_v, fmt,
                                          static_cast<hipStream_t>(stream)),
                    "gdn_qdq_state launch");
}

}  // extern "C"
