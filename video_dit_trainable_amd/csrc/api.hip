// C-ABI entry points of libvsa2 (declared in include/vsa2.h): argument
// validation, workspace carving and kernel launches.  No allocation, no
// synchronisation; every call enqueues on the caller's stream.
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/vsa2.h"
#include "launch.h"

using namespace vsa2;

namespace {

constexpr size_t ALIGN = 256;
constexpr int MAX_DEVICES_GRID = 64;

size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

// nb counts attention blocks (the rows and columns of the router scores and
// of the selection, the coarse tokens), nc the 4x4x4 cubes the kernels tile
// over; nb = nc >> bs with 2^bs cubes per block.
struct Dims {
  int batch, heads, bh, d, L, nb, nbp, Lr;  // Lr: router rows per head in the pooled buffer
  int rp;                                    // router pool edge: 1, 2 or 4
  int nc, bs;
  int nt, ntc, ld;  // MMDiT text tokens, their 64-row cubes, token rows per head (L + 64 ntc)
  bool bf16;
  size_t esz;
  float scale;
  PadGrid pad;
};

int check_problem(const vsa2_problem* p, Dims& o) {
  if (!p) return VSA2_E_ARG;
  if (p->batch < 1 || p->heads < 1) return VSA2_E_SHAPE;
  if (p->head_dim != 64 && p->head_dim != 128) return VSA2_E_SHAPE;
  if (p->lat_t < 1 || p->lat_y < 1 || p->lat_x < 1) return VSA2_E_SHAPE;
  if (p->lat_t > (1 << 20) || p->lat_y > (1 << 20) || p->lat_x > (1 << 20)) return VSA2_E_SHAPE;
  if (p->dtype != VSA2_F32 && p->dtype != VSA2_BF16) return VSA2_E_ARG;
  if (p->block_tokens != 0 && p->block_tokens != 64 && p->block_tokens != 128) return VSA2_E_SHAPE;
  if (p->text_tokens < 0 || p->text_tokens > (1 << 20)) return VSA2_E_SHAPE;
  if (p->router_pool != 0 && p->router_pool != 1 && p->router_pool != 2 && p->router_pool != 4) return VSA2_E_SHAPE;
  const int bs = p->block_tokens == 128 ? 1 : 0;  // a 128-token block is two x-adjacent cubes
  // a grid that is not a whole number of blocks is padded up to one
  const int64_t xs = 4 << bs;
  const int64_t nt = (p->lat_t + 3) / 4, ny = (p->lat_y + 3) / 4, nx = (p->lat_x + xs - 1) / xs << bs;
  const int64_t nc = nt * ny * nx;
  const int64_t L = 64 * nc;
  if (nc > 46340) return VSA2_E_SHAPE;  // nc^2 and all indices fit int32
  const int64_t nb = nc >> bs;
  // launch limits: (batch, head) pairs index grid.y (at most 65,535), and the
  // largest one-dimensional grid, about (cubes + text cubes + 8) workgroups of
  // 256 threads per (batch, head), must keep its work-item count within 32 bits
  const int64_t bh = (int64_t)p->batch * p->heads;
  if (bh > 65535) return VSA2_E_SHAPE;
  const int64_t ntc = ((int64_t)p->text_tokens + 63) / 64;
  if (bh * (8 * ((nc + 7) / 8) + ntc + 8) * 256 > (int64_t)0xFFFFFFFF) return VSA2_E_SHAPE;
  if (std::isnan(p->softmax_scale) || std::isinf(p->softmax_scale)) return VSA2_E_ARG;
  o.batch = p->batch;
  o.heads = p->heads;
  o.bh = p->batch * p->heads;
  o.d = p->head_dim;
  o.L = (int)L;
  o.nb = (int)nb;
  o.nbp = (int)((nb + 63) / 64 * 64);
  o.nc = (int)nc;
  o.bs = bs;
  o.nt = p->text_tokens;
  o.ntc = (p->text_tokens + 63) / 64;
  o.ld = o.L + 64 * o.ntc;
  o.rp = p->router_pool ? p->router_pool : 2;
  o.Lr = o.rp == 1 ? (int)L : (o.rp == 2 ? (int)(L / 8) : 0);  // pool 4 routes on Q_c, K_c
  o.bf16 = p->dtype == VSA2_BF16;
  o.esz = o.bf16 ? 2 : 4;
  o.scale = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / std::sqrt((float)p->head_dim);
  o.pad.on = (p->lat_t % 4) || (p->lat_y % 4) || (p->lat_x % xs);
  o.pad.nt = (int)nt;
  o.pad.ny = (int)ny;
  o.pad.nx = (int)nx;
  o.pad.rt = p->lat_t;
  o.pad.ry = p->lat_y;
  o.pad.rx = p->lat_x;
  o.pad.inv_nx = (float)(1.0 / (double)nx);
  o.pad.inv_nyx = (float)(1.0 / (double)(ny * nx));
  return VSA2_OK;
}

bool aligned(const void* ptr) { return ptr && ((uintptr_t)ptr % 16 == 0); }

// The CSC outputs of the TopK calls: both given (aligned), or both NULL for a
// forward-only selection (no CSC, and only the query side of the schedule).
bool csc_args_ok(const int32_t* col_ptr, const int32_t* row_idx) {
  if (!col_ptr && !row_idx) return true;
  return aligned(col_ptr) && aligned(row_idx);
}

int64_t budget(const Dims& d, int32_t topk) {
  const int64_t all = (int64_t)d.nb * d.nb;
  const int64_t k = (int64_t)d.nb * topk;
  return k < all ? k : all;
}

int bitmap_words(const Dims& d) { return 2 * ((d.nb + 63) / 64); }

// Workspace layouts --------------------------------------------------------
// per-row LSE, then (padded grids) one existence word per 64 pooled keys
// pool 1: then the 8 x 8 sub-cube means [bh, 8 nc, 8 nc]; pool 4: the LSE of the
// coarse rows (as vsa2_route_coarse)
size_t ws_route_lse(const Dims& d) { return up((size_t)d.bh * (d.rp == 4 ? d.nb : d.Lr) * 4); }
size_t ws_route(const Dims& d) {
  if (d.rp == 1) return ws_route_lse(d) + up((size_t)d.bh * 64 * d.nc * d.nc * 4);
  return ws_route_lse(d) + (d.pad.on ? up((size_t)(d.Lr + 63) / 64 * 8) : 0);
}

size_t ws_topk(const Dims& d, TopkWs* w, void* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up(bytes);
    return o;
  };
  const size_t o_hist = take((size_t)d.bh * 4096 * 4);
  const size_t o_state = take((size_t)d.bh * 16);
  const size_t o_row = take((size_t)d.bh * 2 * d.nb * 4);
  const size_t o_take = take((size_t)d.bh * d.nb * 4);
  const size_t o_col = take((size_t)d.bh * d.nb * 4);
  const size_t o_bm = take((size_t)d.bh * d.nb * bitmap_words(d) * 4);
  const size_t o_sk = take((size_t)2 * d.bh * d.nb * 4);  // the schedule's arrays: both sides
  const size_t o_so = take((size_t)2 * d.bh * d.nb * 4);
  const size_t o_st = take((size_t)2 * d.bh * d.nb * 4);
  const size_t o_sc = take((size_t)2 * d.bh * 8 * 4);
  const size_t o_sh = take((size_t)2 * d.bh * 8 * 4);
  const size_t o_sp = take((size_t)2 * d.bh * d.nb);
  const size_t o_sr = take((size_t)2 * d.bh * 9 * 4);
  if (w) {
    char* b = (char*)base;
    w->spx = (uint8_t*)(b + o_sp);
    w->srng = (int32_t*)(b + o_sr);
    w->skeys = (uint32_t*)(b + o_sk);
    w->sorder = (int32_t*)(b + o_so);
    w->stmp = (int32_t*)(b + o_st);
    w->scnt = (int32_t*)(b + o_sc);
    w->shoff = (int32_t*)(b + o_sh);
    w->hist = (uint32_t*)(b + o_hist);
    w->state = (uint32_t*)(b + o_state);
    w->rowcnt = (uint32_t*)(b + o_row);
    w->take = (uint32_t*)(b + o_take);
    w->colcnt = (uint32_t*)(b + o_col);
    w->bitmap = (uint32_t*)(b + o_bm);
    w->words = bitmap_words(d);
  }
  return off;
}

size_t ws_plan(const Dims& d, TopkWs* w, void* base) {
  const size_t o_col = 0;
  const size_t o_bm = up((size_t)d.bh * d.nb * 4);
  const size_t o_sk = o_bm + up((size_t)d.bh * d.nb * bitmap_words(d) * 4);  // the schedule's: both sides
  const size_t o_so = o_sk + up((size_t)2 * d.bh * d.nb * 4);
  const size_t o_st = o_so + up((size_t)2 * d.bh * d.nb * 4);
  const size_t o_sc = o_st + up((size_t)2 * d.bh * d.nb * 4);
  const size_t o_sh = o_sc + up((size_t)2 * d.bh * 8 * 4);
  const size_t o_sp = o_sh + up((size_t)2 * d.bh * 8 * 4);
  const size_t o_sr = o_sp + up((size_t)2 * d.bh * d.nb);
  if (w) {
    char* b = (char*)base;
    *w = TopkWs{};
    w->colcnt = (uint32_t*)(b + o_col);
    w->bitmap = (uint32_t*)(b + o_bm);
    w->words = bitmap_words(d);
    w->skeys = (uint32_t*)(b + o_sk);
    w->sorder = (int32_t*)(b + o_so);
    w->stmp = (int32_t*)(b + o_st);
    w->scnt = (int32_t*)(b + o_sc);
    w->shoff = (int32_t*)(b + o_sh);
    w->spx = (uint8_t*)(b + o_sp);
    w->srng = (int32_t*)(b + o_sr);
  }
  return o_sr + up((size_t)2 * d.bh * 9 * 4);
}

// The fine branch's work schedule (sched.hip): the fine kernels run one
// attention block (a cube, or a whole 128-token block) per work item, and
// with text rows one text cube per further item (64-token blocks only: with
// 128-token blocks and text rows the kernels run per cube, and there is no
// schedule).  Layout: for the query blocks, then for the KV blocks, a 256-byte
// header (queue starts and lengths, item count, marker) and the items
// [bh * (nb + ntc)] int32 (nb attention blocks, ntc text cubes).
bool sched_on(const Dims& d) { return d.ntc == 0 || d.bs == 0; }
struct SchedPtrs {
  int32_t *rh, *ri, *ch, *ci;
};
size_t sched_layout(const Dims& d, int64_t k, const void* base, SchedPtrs* sp) {
  (void)k;
  if (!sched_on(d)) return 0;
  const size_t side = ALIGN + up((size_t)d.bh * (d.nb + d.ntc) * 4);
  if (sp) {
    char* b = (char*)base;
    sp->rh = (int32_t*)b;
    sp->ri = (int32_t*)(b + ALIGN);
    sp->ch = (int32_t*)(b + side);
    sp->ci = (int32_t*)(b + side + ALIGN);
  }
  return 2 * side;
}
size_t ws_fwd(const Dims& d) { return sched_on(d) ? ALIGN : 0; }

// Checks a caller's schedule buffer: NULL is allowed (no schedule: one
// workgroup per cube in the natural order); otherwise aligned and, when its
// size is known, large enough.
int check_sched(const Dims& d, int64_t k, const void* sched, const size_t* bytes) {
  const size_t need = sched_layout(d, k, nullptr, nullptr);
  if (!sched || need == 0) return VSA2_OK;
  if ((uintptr_t)sched % ALIGN) return VSA2_E_ARG;
  if (bytes && *bytes < need) return VSA2_E_WORKSPACE;
  return VSA2_OK;
}
// Builds the schedule into `sched` (when there is one) from the selection's
// CSR and CSC.
hipError_t build_sched(const Dims& d, int64_t k, const TopkArgs& a, void* sched, hipStream_t st) {
  if (!sched || !sched_on(d)) return hipSuccess;
  SchedPtrs sp;
  sched_layout(d, k, sched, &sp);
  SchedArgs s{a.row_ptr, a.col_idx, a.col_ptr, a.row_idx, sp.rh, sp.ri, sp.ch, sp.ci, a.ws.skeys, a.ws.sorder,
              a.ws.stmp, a.ws.scnt, a.ws.shoff, a.ws.spx, a.ws.srng, d.bh, d.nb, k, d.ntc};
  return launch_sched(s, st);
}

// (lse2, delta) per token row, then the schedule's queue counters (8 for the
// dQ pass, 8 for the dK/dV pass)
size_t ws_bwd_stats(const Dims& d) { return up((size_t)d.bh * d.ld * 8); }
size_t ws_bwd(const Dims& d) { return ws_bwd_stats(d) + ALIGN; }

size_t ws_fwd(const Dims& d);  // the schedule's 8 queue counters (below)


int pad16(int x) { return (x + 15) / 16 * 16; }
int pad32(int x) { return (x + 31) / 32 * 32; }

size_t wt_bytes(const Dims& d, int dm) { return up((size_t)(2 * pad16(d.heads) + 2 * pad32(d.heads)) * dm * d.esz); }

int nchunk_of(const Dims& d) { return (d.L + DW_TC - 1) / DW_TC; }

struct CoarseBwdWs {
  void* wt;
  float* dpre;
  void* doc;
  float* stats_c;
  float* dw_part;
  float* doc_part;  // 128-token blocks: per-cube sums of dO_hat_c
};

size_t ws_coarse_bwd(const Dims& d, int dm, CoarseBwdWs* w, void* base) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up(bytes);
    return o;
  };
  const size_t o_wt = take(wt_bytes(d, dm));
  const size_t o_dpre = take((size_t)d.bh * d.L * 4);
  const size_t o_doc = take((size_t)d.bh * d.nbp * d.d * d.esz);
  const size_t o_dc = take((size_t)d.bh * d.nbp * 8);
  const size_t o_dw = take((size_t)d.batch * nchunk_of(d) * dm * d.heads * 4);
  const size_t o_dp = take(d.bs ? (size_t)d.bh * d.nc * d.d * 4 : 0);
  if (w) {
    char* b = (char*)base;
    w->wt = b + o_wt;
    w->dpre = (float*)(b + o_dpre);
    w->doc = b + o_doc;
    w->stats_c = (float*)(b + o_dc);
    w->dw_part = (float*)(b + o_dw);
    w->doc_part = d.bs ? (float*)(b + o_dp) : nullptr;
  }
  return off;
}

int check_dm(const Dims& d, int32_t dm) {
  if (dm < 64 || dm % 64) return VSA2_E_SHAPE;
  if (d.heads > 64) return VSA2_E_UNSUPPORTED;
  return VSA2_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return VSA2_OK;
  if (!ws || ((uintptr_t)ws % ALIGN)) return ws ? VSA2_E_ARG : VSA2_E_WORKSPACE;
  return have >= need ? VSA2_OK : VSA2_E_WORKSPACE;
}

int hip_status(hipError_t e) { return e == hipSuccess ? VSA2_OK : VSA2_E_HIP; }

struct Pooled {
  const void *qr, *kr, *qc, *kc, *vc;
};
Pooled pooled_ptrs(const Dims& d, const void* base) {
  const char* b = (const char*)base;
  const size_t r = (size_t)d.bh * d.Lr * d.d * d.esz;
  const size_t c = (size_t)d.bh * d.nbp * d.d * d.esz;
  return Pooled{b, b + r, b + 2 * r, b + 2 * r + c, b + 2 * r + 2 * c};
}

// Pools 1 and 4 serve 64-token blocks on unpadded grids; pool 1's sub-cube
// intermediate has (8 nc)^2 entries per head, kept within int32 indices.
bool route_supported(const Dims& d) {
  if (d.rp == 2) return true;
  if (d.pad.on || d.bs) return false;
  return d.rp == 4 || 8 * (int64_t)d.nc <= 46340;
}

// The router launches of vsa2_route / vsa2_route_noalloc for every pool.
hipError_t route_launch(const Dims& d, const void* pooled, float* scores, void* ws, hipStream_t st) {
  Pooled pp = pooled_ptrs(d, pooled);
  const float sl2 = d.scale * 1.4426950408889634f;
  if (d.rp == 4) {  // one pooled token per cube: the coarse operands, and P_r = P_c
    RouteArgs a{pp.qc, pp.kc, (float*)ws, scores, d.bh, d.nb, d.d, d.bf16, sl2, PadGrid{}, nullptr, 0, 1, d.nbp};
    return launch_route(a, st);
  }
  if (d.rp == 1) {  // every token: 8 x 8 means over sub-cube pairs, then 8 x 8 blocks of those
    float* sub = (float*)((char*)ws + ws_route_lse(d));
    RouteArgs a{pp.qr, pp.kr, (float*)ws, sub, d.bh, 8 * d.nc, d.d, d.bf16, sl2, PadGrid{}, nullptr, 0};
    hipError_t e = launch_route(a, st);
    if (e != hipSuccess) return e;
    return launch_route_fold(sub, scores, d.bh, d.nc, st);
  }
  RouteArgs a{pp.qr, pp.kr, (float*)ws, scores, d.bh, d.nc, d.d, d.bf16, sl2, d.pad,
              d.pad.on ? (uint64_t*)((char*)ws + ws_route_lse(d)) : nullptr, d.bs};
  return launch_route(a, st);
}

// Diagnostic kernel timer ----------------------------------------------------
struct KernelTimer {
  bool armed = false;
  int capacity = 0, used = 0;
  hipEvent_t ev[2 * 4096];
  int created = 0;
};
KernelTimer g_timer[VSA2_K_COUNT];

}  // namespace

namespace vsa2 {
int resident_grid(const void* fn, int threads, int items) {
  static std::mutex mu;
  static int cus[MAX_DEVICES_GRID] = {};
  int dev = 0;
  (void)hipGetDevice(&dev);
  int n_cu = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < MAX_DEVICES_GRID) {
      if (!cus[dev]) (void)hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev);
      n_cu = cus[dev];
    }
  }
  int per = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, threads, 0) != hipSuccess || per < 1) per = 1;
  if (n_cu < 1) n_cu = 8;
  long g = (long)n_cu * per;
  const long cap = ((long)items + 7) / 8 * 8;
  if (g > cap) g = cap;
  g = (g + 7) / 8 * 8;
  return (int)(g < 8 ? 8 : g);
}

void timer_before(int kid, hipStream_t st) {
  KernelTimer& t = g_timer[kid];
  if (!t.armed || t.used >= t.capacity) return;
  const int i = 2 * t.used;
  while (t.created < i + 2) {
    if (hipEventCreate(&t.ev[t.created]) != hipSuccess) { t.armed = false; return; }
    ++t.created;
  }
  (void)hipEventRecord(t.ev[i], st);
}
void timer_after(int kid, hipStream_t st) {
  KernelTimer& t = g_timer[kid];
  if (!t.armed || t.used >= t.capacity) return;
  (void)hipEventRecord(t.ev[2 * t.used + 1], st);
  ++t.used;
}
}  // namespace vsa2

// Fixed device scratch of the no-allocation router entry point: one copy of
// this array lives on every GPU the library runs on, for the life of the
// process.  Host code never passes the array's name to a kernel (on the host
// it names a stand-in, not device memory): its device address is looked up
// once per device with hipGetSymbolAddress and that address is used instead.
constexpr size_t SCRATCH_BYTES = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of `scratch` on the current device, looked up on the first
// call for that device.  Returns hipSuccess and the address, or the error of
// hipGetDevice / hipGetSymbolAddress.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr || (uintptr_t)ptr % ALIGN) return hipErrorInvalidValue;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

int vsa2_kernel_timer_start(int32_t kernel, int32_t capacity) {
  if (kernel < 0 || kernel >= VSA2_K_COUNT || capacity < 1 || capacity > 4096) return VSA2_E_ARG;
  KernelTimer& t = g_timer[kernel];
  t.armed = true;
  t.capacity = capacity;
  t.used = 0;
  return VSA2_OK;
}

int vsa2_kernel_timer_stop(int32_t kernel, float* ms, int32_t* launches) {
  if (kernel < 0 || kernel >= VSA2_K_COUNT || !ms || !launches) return VSA2_E_ARG;
  KernelTimer& t = g_timer[kernel];
  float sum = 0.f;
  int status = VSA2_OK;
  if (t.used > 0 && hipEventSynchronize(t.ev[2 * t.used - 1]) != hipSuccess) status = VSA2_E_HIP;
  for (int i = 0; status == VSA2_OK && i < t.used; ++i) {
    float x = 0.f;
    if (hipEventElapsedTime(&x, t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess) status = VSA2_E_HIP;
    sum += x;
  }
  *ms = sum;
  *launches = t.used;
  t.armed = false;
  t.used = 0;
  return status;
}

const char* vsa2_status_string(int s) {
  switch (s) {
    case VSA2_OK: return "ok";
    case VSA2_E_ARG: return "invalid argument (NULL/misaligned pointer or bad scalar)";
    case VSA2_E_SHAPE: return "unsupported shape (empty or oversized grid, head_dim not 64 or 128)";
    case VSA2_E_WORKSPACE: return "workspace too small";
    case VSA2_E_HIP: return "HIP launch failed";
    case VSA2_E_UNSUPPORTED: return "unsupported request";
    case VSA2_E_SCRATCH: return "problem needs more scratch than the no-allocation entry point's fixed device array";
    default: return "unknown status";
  }
}

int vsa2_budget(const vsa2_problem* p, int32_t topk, int64_t* k) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (!k || topk < 1) return VSA2_E_ARG;
  *k = budget(d, topk);
  return VSA2_OK;
}

int vsa2_sched_size(const vsa2_problem* p, int32_t topk, size_t* bytes) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (!bytes || topk < 1) return VSA2_E_ARG;
  *bytes = sched_layout(d, budget(d, topk), nullptr, nullptr);
  return VSA2_OK;
}

int vsa2_pooled_size(const vsa2_problem* p, size_t* bytes) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (!bytes) return VSA2_E_ARG;
  *bytes = (size_t)d.bh * (2 * (size_t)d.Lr + 3 * (size_t)d.nbp) * d.d * d.esz;
  return VSA2_OK;
}

int vsa2_saved_size(const vsa2_problem* p, size_t* bytes) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (!bytes) return VSA2_E_ARG;
  *bytes = ((size_t)d.bh * d.nb * d.d + (size_t)d.bh * d.nb + (size_t)d.bh * d.L) * 4;
  return VSA2_OK;
}

int vsa2_workspace_size(const vsa2_problem* p, int32_t op, int32_t topk, int32_t d_model, size_t* bytes) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (!bytes) return VSA2_E_ARG;
  switch (op) {
    case VSA2_OP_POOL: *bytes = 0; break;
    case VSA2_OP_ROUTE: *bytes = ws_route(d); break;
    case VSA2_OP_TOPK: *bytes = ws_topk(d, nullptr, nullptr); break;
    case VSA2_OP_PLAN: *bytes = ws_plan(d, nullptr, nullptr); break;
    case VSA2_OP_FWD: *bytes = ws_fwd(d); break;
    case VSA2_OP_BWD: *bytes = ws_bwd(d); break;
    case VSA2_OP_COARSE:
      if ((s = check_dm(d, d_model))) return s;
      *bytes = wt_bytes(d, d_model);
      break;
    case VSA2_OP_COARSE_BWD:
      if ((s = check_dm(d, d_model))) return s;
      *bytes = ws_coarse_bwd(d, d_model, nullptr, nullptr);
      break;
    case VSA2_OP_ROUTE_COARSE: *bytes = up((size_t)d.bh * d.nb * 4); break;
    case VSA2_OP_TOPK_ROW: *bytes = ws_plan(d, nullptr, nullptr); break;
    default: return VSA2_E_ARG;
  }
  (void)topk;
  return VSA2_OK;
}

int vsa2_pool(const vsa2_problem* p, const void* q, const void* k, const void* v, void* pooled, void* stream) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (!route_supported(d)) return VSA2_E_UNSUPPORTED;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(pooled)) return VSA2_E_ARG;
  Pooled pp = pooled_ptrs(d, pooled);
  PoolArgs a{q, k, v, (void*)pp.qr, (void*)pp.kr, (void*)pp.qc, (void*)pp.kc, (void*)pp.vc, d.bh, d.nc, d.nbp, d.d,
             d.bf16, d.pad, d.bs, d.ld, d.rp};
  return hip_status(launch_pool(a, (hipStream_t)stream));
}

int vsa2_route(const vsa2_problem* p, const void* pooled, float* scores, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (!route_supported(d)) return VSA2_E_UNSUPPORTED;
  if (!aligned(pooled) || !aligned(scores)) return VSA2_E_ARG;
  if ((s = check_ws(ws, ws_bytes, ws_route(d)))) return s;
  return hip_status(route_launch(d, pooled, scores, ws, (hipStream_t)stream));
}

int vsa2_route_noalloc(const vsa2_problem* p, const void* pooled, float* scores, void* stream) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (!aligned(pooled) || !aligned(scores)) return VSA2_E_ARG;
  if (!route_supported(d)) return VSA2_E_UNSUPPORTED;
  const size_t need = ws_route(d);
  if (need > SCRATCH_BYTES) return VSA2_E_SCRATCH;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return VSA2_E_HIP;
  // the router's scratch is written before it is read (the per-row LSE by
  // pass 1, the key-existence words by their own kernel, pool 1's sub-cube
  // means by pass 2), so nothing is cleared
  return hip_status(route_launch(d, pooled, scores, ws, (hipStream_t)stream));
}

int vsa2_route_noalloc_limit(size_t* bytes) {
  if (!bytes) return VSA2_E_ARG;
  *bytes = SCRATCH_BYTES;
  return VSA2_OK;
}

int vsa2_route_coarse(const vsa2_problem* p, const void* pooled, float* scores, void* ws, size_t ws_bytes,
                      void* stream) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (!aligned(pooled) || !aligned(scores)) return VSA2_E_ARG;
  if ((s = check_ws(ws, ws_bytes, up((size_t)d.bh * d.nb * 4)))) return s;
  Pooled pp = pooled_ptrs(d, pooled);
  RouteArgs a{pp.qc, pp.kc, (float*)ws, scores, d.bh, d.nb, d.d, d.bf16, d.scale * 1.4426950408889634f, PadGrid{},
              nullptr, 0, 1, d.nbp};
  return hip_status(launch_route(a, (hipStream_t)stream));
}

int vsa2_topk_per_row(const vsa2_problem* p, const float* scores, int32_t topk, int32_t* row_ptr,
                      int32_t* col_idx, int32_t* col_ptr, int32_t* row_idx, void* sched, size_t sched_bytes,
                      void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (topk < 1) return VSA2_E_ARG;
  if (!aligned(scores) || !aligned(row_ptr) || !aligned(col_idx)) return VSA2_E_ARG;
  if (!csc_args_ok(col_ptr, row_idx)) return VSA2_E_ARG;
  if ((s = check_sched(d, budget(d, topk), sched, &sched_bytes))) return s;
  if ((s = check_ws(ws, ws_bytes, ws_plan(d, nullptr, nullptr)))) return s;
  TopkArgs a{};
  a.scores = scores;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.col_ptr = col_ptr;
  a.row_idx = row_idx;
  a.bh = d.bh;
  a.nb = d.nb;
  a.k = budget(d, topk);  // nb min(topk, nb)
  ws_plan(d, &a.ws, ws);
  hipError_t e = launch_topk_rows(a, (hipStream_t)stream);
  if (e == hipSuccess) e = build_sched(d, a.k, a, sched, (hipStream_t)stream);
  return hip_status(e);
}

int vsa2_topk_per_seq(const vsa2_problem* p, const float* scores, int32_t topk, int32_t* row_ptr, int32_t* col_idx,
                      int32_t* col_ptr, int32_t* row_idx, void* sched, size_t sched_bytes, void* ws,
                      size_t ws_bytes, void* stream) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (topk < 1) return VSA2_E_ARG;
  if (!aligned(scores) || !aligned(row_ptr) || !aligned(col_idx)) return VSA2_E_ARG;
  if (!csc_args_ok(col_ptr, row_idx)) return VSA2_E_ARG;
  if ((s = check_sched(d, budget(d, topk), sched, &sched_bytes))) return s;
  if ((s = check_ws(ws, ws_bytes, ws_topk(d, nullptr, nullptr)))) return s;
  TopkArgs a{};
  a.scores = scores;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.col_ptr = col_ptr;
  a.row_idx = row_idx;
  a.bh = d.bh;
  a.nb = d.nb;
  a.k = budget(d, topk);
  ws_topk(d, &a.ws, ws);
  hipError_t e = launch_topk(a, (hipStream_t)stream);
  if (e == hipSuccess) e = build_sched(d, a.k, a, sched, (hipStream_t)stream);
  return hip_status(e);
}

int vsa2_plan_from_csr(const vsa2_problem* p, int32_t topk, const int32_t* row_ptr, const int32_t* col_idx,
                       int32_t* col_ptr, int32_t* row_idx, void* sched, size_t sched_bytes, void* ws,
                       size_t ws_bytes, void* stream) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (topk < 1) return VSA2_E_ARG;
  if (!aligned(row_ptr) || !aligned(col_idx) || !aligned(col_ptr) || !aligned(row_idx)) return VSA2_E_ARG;
  if ((s = check_sched(d, budget(d, topk), sched, &sched_bytes))) return s;
  if ((s = check_ws(ws, ws_bytes, ws_plan(d, nullptr, nullptr)))) return s;
  TopkArgs a{};
  a.row_ptr = const_cast<int32_t*>(row_ptr);
  a.col_idx = const_cast<int32_t*>(col_idx);
  a.col_ptr = col_ptr;
  a.row_idx = row_idx;
  a.bh = d.bh;
  a.nb = d.nb;
  a.k = budget(d, topk);
  ws_plan(d, &a.ws, ws);
  hipError_t e = launch_plan(a, (hipStream_t)stream);
  if (e == hipSuccess) e = build_sched(d, a.k, a, sched, (hipStream_t)stream);
  return hip_status(e);
}

int vsa2_sparse_attn_fwd(const vsa2_problem* p, int32_t topk, const void* q, const void* k, const void* v,
                         const int32_t* row_ptr, const int32_t* col_idx, const void* sched, void* o_f, float* lse,
                         void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (topk < 1) return VSA2_E_ARG;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(row_ptr) || !aligned(col_idx) || !aligned(o_f) ||
      !aligned(lse))
    return VSA2_E_ARG;
  if ((s = check_sched(d, budget(d, topk), sched, nullptr))) return s;
  if ((s = check_ws(ws, ws_bytes, ws_fwd(d)))) return s;
  AttnArgs a{};
  if (sched && sched_on(d)) {
    SchedPtrs sp;
    sched_layout(d, budget(d, topk), sched, &sp);
    a.sq_hdr = sp.rh;
    a.sq_items = sp.ri;
    a.sq_ctr = (int32_t*)ws;
  }
  a.q = q; a.k = k; a.v = v;
  a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.o = o_f; a.lse = lse;
  a.bh = d.bh; a.nq = d.nc; a.nkv = d.nc; a.seq = d.ld; a.ld = d.ld; a.out_rows = d.ld;
  a.kph = budget(d, topk);
  a.d = d.d; a.bf16 = d.bf16; a.dense = false;
  a.scale_log2 = d.scale * 1.4426950408889634f;
  a.ct = d.pad.nt; a.cy = d.pad.ny; a.cx = d.pad.nx;
  a.pad = d.pad;
  a.bs = d.bs;
  a.ntc = d.ntc; a.ntext = d.nt;
  return hip_status(launch_attn_fwd(a, (hipStream_t)stream));
}

int vsa2_sparse_attn_bwd(const vsa2_problem* p, int32_t topk, const void* q, const void* k, const void* v,
                         const void* o_f, const float* lse, const void* d_o, const int32_t* row_ptr,
                         const int32_t* col_idx, const int32_t* col_ptr, const int32_t* row_idx, const void* sched,
                         const float* dqkv_c, void* dq, void* dk, void* dv, void* ws, size_t ws_bytes,
                         void* stream) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if (topk < 1) return VSA2_E_ARG;
  if (!aligned(q) || !aligned(k) || !aligned(v) || !aligned(o_f) || !aligned(lse) || !aligned(d_o) ||
      !aligned(row_ptr) || !aligned(col_idx) || !aligned(col_ptr) || !aligned(row_idx) || !aligned(dq) ||
      !aligned(dk) || !aligned(dv))
    return VSA2_E_ARG;
  if (dqkv_c && !aligned(dqkv_c)) return VSA2_E_ARG;
  if ((s = check_sched(d, budget(d, topk), sched, nullptr))) return s;
  if ((s = check_ws(ws, ws_bytes, ws_bwd(d)))) return s;
  const hipStream_t st = (hipStream_t)stream;
  AttnBwdArgs a{};
  if (sched && sched_on(d)) {
    SchedPtrs sp;
    sched_layout(d, budget(d, topk), sched, &sp);
    a.sq_hdr = sp.rh;
    a.sq_items = sp.ri;
    a.sk_hdr = sp.ch;
    a.sk_items = sp.ci;
    a.sq_ctr = (int32_t*)((char*)ws + ws_bwd_stats(d));
  }
  a.q = q; a.k = k; a.v = v; a.o = o_f; a.d_o = d_o;
  a.lse = lse;
  a.stats_out = (float*)ws;
  a.row_ptr = row_ptr; a.col_idx = col_idx; a.col_ptr = col_ptr; a.row_idx = row_idx;
  const size_t cstride = (size_t)d.bh * d.nb * d.d;
  a.dq_add = dqkv_c;
  a.dk_add = dqkv_c ? dqkv_c + cstride : nullptr;
  a.dv_add = dqkv_c ? dqkv_c + 2 * cstride : nullptr;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.bh = d.bh; a.nq = d.nc; a.nkv = d.nc; a.seq = d.ld; a.ld = d.ld; a.out_rows = d.ld;
  a.kph = budget(d, topk);
  a.d = d.d; a.bf16 = d.bf16; a.dense = false;
  a.scale = d.scale;
  a.scale_log2 = d.scale * 1.4426950408889634f;
  a.ct = d.pad.nt; a.cy = d.pad.ny; a.cx = d.pad.nx;
  a.pad = d.pad;
  a.bs = d.bs;
  a.ntc = d.ntc; a.ntext = d.nt;
  return hip_status(launch_attn_bwd(a, st));
}

int vsa2_coarse_gate(const vsa2_problem* p, const void* pooled, const void* x, int32_t d_model, const float* w_g,
                     const void* o_f, void* o, float* saved, void* ws, size_t ws_bytes, void* stream) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if ((s = check_dm(d, d_model))) return s;
  if (!aligned(pooled) || !aligned(x) || !aligned(w_g) || !aligned(o_f) || !aligned(o) || !aligned(saved))
    return VSA2_E_ARG;
  if ((s = check_ws(ws, ws_bytes, wt_bytes(d, d_model)))) return s;
  const hipStream_t st = (hipStream_t)stream;
  Pooled pp = pooled_ptrs(d, pooled);
  float* oc_hat = saved;
  float* lse_c = oc_hat + (size_t)d.bh * d.nb * d.d;
  float* g = lse_c + (size_t)d.bh * d.nb;
  AttnArgs a{};
  a.q = pp.qc; a.k = pp.kc; a.v = pp.vc;
  a.o = oc_hat; a.lse = lse_c;
  a.bh = d.bh; a.nq = d.nbp / 64; a.nkv = d.nbp / 64; a.seq = d.nb; a.ld = d.nbp; a.out_rows = d.nb;
  a.kph = 0;
  a.d = d.d; a.bf16 = d.bf16; a.dense = true;
  a.scale_log2 = d.scale * 1.4426950408889634f;
  hipError_t e = launch_attn_fwd(a, st);
  if (e != hipSuccess) return VSA2_E_HIP;
  GateArgs ga{x, w_g, ws, oc_hat, o_f, o, g, d.batch, d.heads, d.nc, d.d, d_model, d.bf16, d.pad, d.bs, d.ld};
  return hip_status(launch_gate_fwd(ga, st));
}

int vsa2_coarse_gate_bwd(const vsa2_problem* p, const void* pooled, const void* x, int32_t d_model, const float* w_g,
                         const float* saved, const void* d_o, float* dqkv_c, void* dx, float* dw_g, void* ws,
                         size_t ws_bytes, void* stream) {
  Dims d;
  int s = check_problem(p, d);
  if (s) return s;
  if ((s = check_dm(d, d_model))) return s;
  if (!aligned(pooled) || !aligned(x) || !aligned(w_g) || !aligned(saved) || !aligned(d_o) || !aligned(dqkv_c) ||
      !aligned(dx) || !aligned(dw_g))
    return VSA2_E_ARG;
  if ((s = check_ws(ws, ws_bytes, ws_coarse_bwd(d, d_model, nullptr, nullptr)))) return s;
  const hipStream_t st = (hipStream_t)stream;
  CoarseBwdWs w{};
  ws_coarse_bwd(d, d_model, &w, ws);
  Pooled pp = pooled_ptrs(d, pooled);
  const float* oc_hat = saved;
  const float* lse_c = oc_hat + (size_t)d.bh * d.nb * d.d;
  const float* g = lse_c + (size_t)d.bh * d.nb;
  GateBwdArgs ga{x, w_g, w.wt, oc_hat, g, d_o, w.dpre, w.doc, lse_c, w.stats_c, w.dw_part, dx, dw_g,
                 d.batch, d.heads, d.nc, d.nbp, d.d, d_model, nchunk_of(d), d.bf16, d.pad, d.bs, w.doc_part, d.ld};
  hipError_t e = launch_gate_bwd(ga, st);
  if (e != hipSuccess) return VSA2_E_HIP;
  AttnBwdArgs a{};
  a.q = pp.qc; a.k = pp.kc; a.v = pp.vc; a.o = nullptr; a.d_o = w.doc;
  a.lse = nullptr;
  a.stats = w.stats_c;
  const size_t cstride = (size_t)d.bh * d.nb * d.d;
  a.dq = dqkv_c; a.dk = dqkv_c + cstride; a.dv = dqkv_c + 2 * cstride;
  a.bh = d.bh; a.nq = d.nbp / 64; a.nkv = d.nbp / 64; a.seq = d.nb; a.ld = d.nbp; a.out_rows = d.nb;
  a.kph = 0;
  a.d = d.d; a.bf16 = d.bf16; a.dense = true;
  a.scale = d.scale;
  a.scale_log2 = d.scale * 1.4426950408889634f;
  return hip_status(launch_attn_bwd(a, st));
}

}  // extern "C"
