// C ABI of the exact tiled attention library (declared in include/fa.h):
// argument validation, launch planning and the decode workspace.
#include <math.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>

#include "../../include/fa.h"
#include "fa_launch.h"

namespace {

struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};

std::mutex g_ws_mutex;
// Keyed by (device, stream): calls on one stream are ordered by the stream,
// so a buffer is never used by two calls at once.
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

int map_err(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

// A library-owned device buffer of at least `need` bytes for calls on
// `stream` of the current device: grown (by a quarter more than asked) with
// stream-ordered allocation, kept for the next call.  The larger buffer is
// allocated before the old one is released, so a failed allocation returns
// FA_ERR_ALLOC with nothing enqueued and the old buffer still held.
int workspace(hipStream_t stream, size_t need, char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace& w = g_ws[std::make_pair(dev, stream)];
  if (w.bytes < need) {
    const size_t grow = need + need / 4;
    void* fresh = nullptr;
    if (hipMallocAsync(&fresh, grow, stream) != hipSuccess) return FA_ERR_ALLOC;
    // The old buffer is released after every earlier call on this stream
    // (stream order).  Should the release be refused, the buffer is left
    // to the process's end rather than failing this call.
    if (w.ptr != nullptr) (void)hipFreeAsync(w.ptr, stream);
    w.ptr = fresh;
    w.bytes = grow;
  }
  *out = (char*)w.ptr;
  return FA_OK;
}

int check_fwd(const void* q, const void* k, const void* v, const void* o, int B, int Hq, int Hkv,
              int Tq, int Tk, int d, int causal, float scale, bool* empty) {
  if (B < 0 || Hq < 0 || Hkv < 1 || Tq < 0 || Tk < 0) return FA_ERR_SHAPE;
  if (causal < 0 || causal > 2) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  *empty = (B == 0 || Hq == 0 || Tq == 0);
  if (*empty) return FA_OK;
  if (q == nullptr || o == nullptr) return FA_ERR_NULL;
  if (Tk > 0 && (k == nullptr || v == nullptr)) return FA_ERR_NULL;
  // Offsets are formed in 64-bit; per-dimension products that index one
  // (batch, head) plane must stay within int range.
  // K and V of one (batch, head) are addressed through 32-bit byte ranges.
  if ((int64_t)Tq * d * 4 > INT32_MAX || (int64_t)Tk * d * 4 > INT32_MAX) return FA_ERR_SHAPE;
  if ((int64_t)B * Hq > INT32_MAX / 2) return FA_ERR_SHAPE;
  // Query tiles run along grid.y (at most 65535 of them, 32 rows or more each).
  if (Tq > 65535 * 32) return FA_ERR_SHAPE;
  return FA_OK;
}

// Causal offset: row i sees key j iff j <= i + offset (1: top-left, 2:
// bottom-right).
int causal_offset(int causal, int Tq, int Tk) { return causal == 2 ? Tk - Tq : 0; }

fa::FwdParams make_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale) {
  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Tq = Tq;
  p.Tk = Tk;
  p.g = Hq / Hkv;
  p.groups = p.g;
  // Scores become base-2 exponents s * |scale| * log2(e); a negative scale
  // is folded into the sign of q (exact), and |scale| is kept away from 0 so
  // that masked (-inf) scores still map to -inf rather than NaN.  Below
  // 1e-30 every visible probability is exactly 1 in fp32 either way.
  const double a = fabs((double)scale);
  p.c = (float)(fmax(a, 1e-30) * 1.4426950408889634);
  p.negate_q = scale < 0.f ? 1 : 0;
  p.causal_off = causal_offset(causal, Tq, Tk);
  (void)d;
  return p;
}

// Largest workgroup count accepted for a decode call.
constexpr int kMaxDecodeWorkgroups = 1 << 20;

// Workgroups for a decode call: the caller's count, or (0) as many as the
// device keeps resident at once, so that every workgroup starts at launch
// and all of them finish together.  Cached per (device, d, heads per
// workgroup, cache type).  Returns a negative status if the device cannot be
// queried.
int decode_workgroups(int d, int hpw, int kv, int num_splits) {
  if (num_splits > 0) return num_splits < kMaxDecodeWorkgroups ? num_splits : kMaxDecodeWorkgroups;
  static std::mutex mu;
  static std::map<std::pair<int, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -FA_ERR_DEVICE;
  const std::pair<int, int> key(dev, (d * 16 + hpw) * 4 + kv);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  const int w = fa::decode_resident_workgroups(d, hpw, kv);
  if (w <= 0) return -FA_ERR_DEVICE;
  cache[key] = w;
  return w;
}

}  // namespace

namespace fa {

int compute_units() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace fa

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
           int Tq, int Tk, int d, int causal, float scale, void* stream) {
  bool empty = false;
  const int st = check_fwd(q, k, v, o, B, Hq, Hkv, Tq, Tk, d, causal, scale, &empty);
  if (st != FA_OK || empty) return st;
  const fa::FwdParams p = make_fwd(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale);
  return map_err(fa::launch_fwd_bf16(p, d, causal != 0, (hipStream_t)stream));
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int Hq,
               int Hkv, int Tq, int Tk, int d, int causal, float scale, void* stream) {
  bool empty = false;
  const int st = check_fwd(q, k, v, o, B, Hq, Hkv, Tq, Tk, d, causal, scale, &empty);
  if (st != FA_OK || empty) return st;
  const fa::FwdParams p = make_fwd(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale);
  return map_err(fa::launch_fwd_f32(p, d, causal != 0, (hipStream_t)stream));
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, const float* qscale,
               const float* kscale, const float* vscale, void* o, float* lse, int B, int Hq,
               int Hkv, int Tq, int Tk, int d, int causal, float scale, void* stream) {
  bool empty = false;
  const int st = check_fwd(q, k, v, o, B, Hq, Hkv, Tq, Tk, d, causal, scale, &empty);
  if (st != FA_OK || empty) return st;
  if (qscale == nullptr || kscale == nullptr || vscale == nullptr) return FA_ERR_NULL;
  fa::FwdParams p = make_fwd(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, d, causal, scale);
  p.qscale = qscale;
  p.kscale = kscale;
  p.vscale = vscale;
  return map_err(fa::launch_fwd_fp8(p, d, causal != 0, (hipStream_t)stream));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Tq, int Tk,
           int d, int causal, float scale, void* stream) {
  if (B < 0 || Hq < 0 || Hkv < 1 || Tq < 0 || Tk < 0) return FA_ERR_SHAPE;
  if (causal < 0 || causal > 2) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (!isfinite(scale)) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B == 0 || Hq == 0 || (Tq == 0 && Tk == 0)) return FA_OK;
  if (Tq > 0 && (q == nullptr || o == nullptr || lse == nullptr || dout == nullptr || dq == nullptr))
    return FA_ERR_NULL;
  if (Tk > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)) return FA_ERR_NULL;
  // Byte ranges of one (batch, head) plane are 32-bit; workgroup counts
  // (tiles x heads) must fit the grid.
  if ((int64_t)Tq * d * 4 > INT32_MAX || (int64_t)Tk * d * 4 > INT32_MAX) return FA_ERR_SHAPE;
  const int64_t Tqp = ((int64_t)Tq + fa::kBwdRowPad - 1) / fa::kBwdRowPad * fa::kBwdRowPad;
  if ((int64_t)B * Hq * ((Tq + 127) / 128) > INT32_MAX) return FA_ERR_SHAPE;
  if ((int64_t)B * Hkv * ((Tk + 127) / 128) > INT32_MAX) return FA_ERR_SHAPE;
  if ((int64_t)B * Hq * Tqp / 16 > INT32_MAX) return FA_ERR_SHAPE;

  hipStream_t hs = (hipStream_t)stream;
  const size_t rows = (size_t)B * Hq * (size_t)Tqp;
  // Small causal grids split each dK/dV key block over kparts workgroups,
  // whose fp32 partials live in the workspace after the row terms.
  const int kparts = Tk > 0 ? fa::bwd_key_parts(B, Hkv, Tk, causal != 0) : 1;
  const size_t pfl = kparts > 1 ? (size_t)kparts * B * Hkv * (size_t)Tk * d : 0;   // floats per tensor
  char* ws = nullptr;
  if (rows > 0 || pfl > 0) {
    const int wst = workspace(hs, (2 * rows + 2 * pfl) * sizeof(float), &ws);
    if (wst != FA_OK) return wst;
  }
  fa::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.l2 = rows > 0 ? (float*)ws : nullptr;
  p.delta = rows > 0 ? (float*)ws + rows : nullptr;
  p.kparts = kparts;
  p.part_dk = pfl > 0 ? (float*)ws + 2 * rows : nullptr;
  p.part_dv = pfl > 0 ? (float*)ws + 2 * rows + pfl : nullptr;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Tq = Tq;
  p.Tk = Tk;
  p.Tqp = (int)Tqp;
  p.causal_off = causal_offset(causal, Tq, Tk);
  p.g = Hq / Hkv;
  p.c = (float)((double)scale * 1.4426950408889634);
  p.scale = scale;
  return map_err(fa::launch_bwd(p, d, causal != 0, hs));
}

namespace {

int decode_workgroups_checked(int B, int Hq, int Hkv, int Tk_max, int d, int num_splits, int kv) {
  if (B < 0 || Hq < 0 || Hkv < 1 || Tk_max < 0 || num_splits < 0 || Hq % Hkv != 0)
    return -FA_ERR_SHAPE;
  if (d != 64 && d != 128) return -FA_ERR_UNSUPPORTED;
  return decode_workgroups(d, fa::decode_heads_per_workgroup(Hq / Hkv), kv, num_splits);
}

// fixed_ws == nullptr: the workspace comes from the per-(device, stream)
// buffer, grown on demand.  Otherwise it is the caller-provided device
// memory fixed_ws of fixed_cap bytes; a call that needs more returns
// FA_ERR_SCRATCH before anything is enqueued.
int decode_impl(const void* q, const void* kcache, const void* vcache, const float* kscale,
                const float* vscale, const int* seqlens, void* o, int B, int Hq, int Hkv,
                int Tk_max, int d, int num_splits, int kv, void* stream,
                char* fixed_ws = nullptr, size_t fixed_cap = 0) {
  if (B < 0 || Hq < 0 || Hkv < 1 || Tk_max < 0 || num_splits < 0) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B == 0 || Hq == 0) return FA_OK;
  if (q == nullptr || o == nullptr || seqlens == nullptr) return FA_ERR_NULL;
  if (Tk_max > 0 && (kcache == nullptr || vcache == nullptr)) return FA_ERR_NULL;
  const bool codes = kv != fa::kKvBf16;
  if (codes && Tk_max > 0 && (kscale == nullptr || vscale == nullptr)) return FA_ERR_NULL;
  // One merge wavefront per (sequence, query head).
  if ((int64_t)B * Hq > INT32_MAX / 2) return FA_ERR_SHAPE;

  const int g = Hq / Hkv;
  const int hpw = fa::decode_heads_per_workgroup(g);
  const int W = decode_workgroups(d, hpw, kv, num_splits);
  if (W < 0) return -W;
  const size_t slots = fa::decode_slots(W, B, Hkv, g, hpw);
  const size_t cum_bytes = (((size_t)B + 1) * sizeof(long long) + 255) / 256 * 256;
  const size_t nparts = slots * hpw;
  const size_t need = cum_bytes + nparts * (size_t)(d + 2) * sizeof(float);
  hipStream_t hs = (hipStream_t)stream;

  char* ws = fixed_ws;
  if (ws == nullptr) {
    const int wst = workspace(hs, need, &ws);
    if (wst != FA_OK) return wst;
  } else if (need > fixed_cap) {
    return FA_ERR_SCRATCH;
  }

  fa::DecodeParams p{};
  p.q = q;
  p.kcache = kcache;
  p.vcache = vcache;
  p.kscale = codes ? kscale : nullptr;
  p.vscale = codes ? vscale : nullptr;
  p.seqlens = seqlens;
  p.o = o;
  p.cum = (long long*)ws;
  p.part_m = (float*)(ws + cum_bytes);
  p.part_l = p.part_m + nparts;
  p.part_o = p.part_l + nparts;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Tk_max = Tk_max;
  p.g = g;
  p.hpw = hpw;
  p.W = W;
  p.c = (float)(1.4426950408889634 / sqrt((double)d));
  return map_err(fa::launch_decode(p, d, kv, hs));
}

// Workspace of fa_decode_noalloc: a fixed device array in this library's
// code object, one copy per device, held until the process ends.  Host code
// never uses its name as an address (on the host the name is only a stand-in
// for the symbol): the device address of each device's copy is looked up
// once, with that device current, and kept per device.  Every slot the merge
// kernel reads was written earlier in the same call, so nothing in it has to
// start at zero.
static __device__ __align__(256) char scratch[FA_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of the current device's scratch copy, or null with *status
// set (FA_ERR_DEVICE) when the device or the symbol cannot be queried.
char* scratch_address(int* status) {
  static std::mutex mu;
  static char* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = FA_ERR_DEVICE;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      *status = FA_ERR_DEVICE;
      return nullptr;
    }
    addr[dev] = (char*)ptr;
  }
  *status = FA_OK;
  return addr[dev];
}

}  // namespace

int fa_decode_workgroups(int B, int Hq, int Hkv, int Tk_max, int d, int num_splits) {
  return decode_workgroups_checked(B, Hq, Hkv, Tk_max, d, num_splits, fa::kKvBf16);
}

int fa_decode_fp8_workgroups(int B, int Hq, int Hkv, int Tk_max, int d, int num_splits) {
  return decode_workgroups_checked(B, Hq, Hkv, Tk_max, d, num_splits, fa::kKvE4m3);
}

int fa_decode_int8_workgroups(int B, int Hq, int Hkv, int Tk_max, int d, int num_splits) {
  return decode_workgroups_checked(B, Hq, Hkv, Tk_max, d, num_splits, fa::kKvInt8);
}

int fa_decode(const void* q, const void* kcache, const void* vcache, const int* seqlens, void* o,
              int B, int Hq, int Hkv, int Tk_max, int d, int num_splits, void* stream) {
  return decode_impl(q, kcache, vcache, nullptr, nullptr, seqlens, o, B, Hq, Hkv, Tk_max, d,
                     num_splits, fa::kKvBf16, stream);
}

int fa_decode_noalloc(const void* q, const void* kcache, const void* vcache, const int* seqlens,
                      void* o, int B, int Hq, int Hkv, int Tk_max, int d, int num_splits,
                      void* stream) {
  if (B < 0 || Hq < 0 || Hkv < 1 || Tk_max < 0 || num_splits < 0) return FA_ERR_SHAPE;
  if (B == 0 || Hq == 0) return FA_OK;
  int st = FA_OK;
  char* ws = scratch_address(&st);
  if (ws == nullptr) return st;
  return decode_impl(q, kcache, vcache, nullptr, nullptr, seqlens, o, B, Hq, Hkv, Tk_max, d,
                     num_splits, fa::kKvBf16, stream, ws, FA_DECODE_SCRATCH_BYTES);
}

int fa_decode_fp8(const void* q, const void* kcache, const void* vcache, const float* kscale,
                  const float* vscale, const int* seqlens, void* o, int B, int Hq, int Hkv,
                  int Tk_max, int d, int num_splits, void* stream) {
  return decode_impl(q, kcache, vcache, kscale, vscale, seqlens, o, B, Hq, Hkv, Tk_max, d,
                     num_splits, fa::kKvE4m3, stream);
}

int fa_decode_int8(const void* q, const void* kcache, const void* vcache, const float* kscale,
                   const float* vscale, const int* seqlens, void* o, int B, int Hq, int Hkv,
                   int Tk_max, int d, int num_splits, void* stream) {
  return decode_impl(q, kcache, vcache, kscale, vscale, seqlens, o, B, Hq, Hkv, Tk_max, d,
                     num_splits, fa::kKvInt8, stream);
}

int fa_read_probe(const void* src, size_t bytes, unsigned* sink, void* stream) {
  if (bytes % 16 != 0 || bytes / ((size_t)1 << 20) >= (size_t)INT32_MAX) return FA_ERR_SHAPE;
  if (bytes == 0) return FA_OK;
  if (src == nullptr || sink == nullptr) return FA_ERR_NULL;
  return map_err(fa::launch_read_probe(src, bytes, sink, (hipStream_t)stream));
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape or size argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension (64 or 128)";
    case FA_ERR_ALLOC: return "workspace allocation failed";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_DEVICE: return "no usable HIP device";
    case FA_ERR_SCRATCH: return "workspace exceeds the fixed decode scratch (FA_DECODE_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

void fa_release_workspace(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (auto& kv : g_ws) {
    if (kv.second.ptr != nullptr) {
      // hipFree (not the stream-ordered form): the stream a buffer was
      // grown on may no longer exist.
      (void)hipSetDevice(kv.first.first);
      (void)hipFree(kv.second.ptr);
    }
  }
  g_ws.clear();
  (void)hipSetDevice(cur);
}

}  // extern "C"
