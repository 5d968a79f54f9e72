// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa2 {

// Latent grids whose sides are not multiples of the block are padded up to
// whole blocks (paper §2.2 "Kernel Implementation"); pad positions are not
// tokens.  PadGrid gives the cube grid and the real side lengths; a cube's
// real extent along an axis is the side length minus its offset, clamped to
// 0..4 (with 128-token blocks the last cube along x can hold no token).
// `on` is 0 when the grid divides.
struct PadGrid {
  int on;
  int nt, ny, nx;        // cubes along t, y, x
  int rt, ry, rx;        // real side lengths of the latent grid
  float inv_nx, inv_nyx; // 1 / nx, 1 / (ny nx), rounded to nearest
};

struct PoolArgs {
  const void *q, *k, *v;
  void *qr, *kr, *qc, *kc, *vc;
  int bh, nb, nbp, d;     // nb cubes; nbp rows of the coarse operands (blocks rounded up to 64)
  bool bf16;
  PadGrid pad;
  int bs;                 // 2^bs cubes per attention block (coarse token)
  int ld;                 // token rows per head in q/k/v (video slots, then text rows)
  int rp;                 // router pool edge: 2 (sub-cube means), 1 (the tokens), 4 (no router rows)
};
hipError_t launch_pool(const PoolArgs& a, hipStream_t st);

struct RouteArgs {
  const void *qr, *kr;
  float* lse2;        // workspace [bh, 8*nb], log2-domain LSE of each pooled query
  float* scores;      // [bh, nb >> bs, nb >> bs]
  int bh, nb, d;      // nb cubes
  bool bf16;
  float scale_log2;   // softmax scale * log2(e)
  PadGrid pad;
  uint64_t* kmask;    // workspace [ceil(8 nb / 64)] (padded grids): bit b of word t set when pooled key 64t + b exists
  int bs;             // 2^bs cubes per attention block: the scores are means over block pairs
  int g1;             // VSA router baseline: qr, kr are the coarse operands (hstride rows per head), nb counts
  int hstride;        //   blocks, and the scores are P_c itself
};
hipError_t launch_route(const RouteArgs& a, hipStream_t st);
// Router pool 1: scores[bh][c][g] = mean of the 8 x 8 block of sub[bh][8c..][8g..]
// (sub: [bh, 8 nc, 8 nc] means over sub-cube pairs).
hipError_t launch_route_fold(const float* sub, float* scores, int bh, int nc, hipStream_t st);

struct TopkWs {       // carved from the caller workspace
  uint32_t* hist;     // [bh, 4096]
  uint32_t* state;    // [bh, 4]: prefix, need, count above, pad
  uint32_t* rowcnt;   // [bh, 2, nb]: (> tau, == tau) per row
  uint32_t* take;     // [bh, nb] ties taken per row
  uint32_t* colcnt;   // [bh, nb]
  uint32_t* bitmap;   // [bh, nb, words]
  int words;          // 32-bit words per bitmap row (multiple of 2)
  // schedule, both sides (query-cube lists, then KV-cube lists): 2 bh entries
  uint32_t* skeys;    // [2 bh, nb] min-hash key of every list
  int32_t* sorder;    // [2 bh, nb] cubes in key order
  int32_t* stmp;      // [2 bh, nb] cubes in queue order
  int32_t* scnt;      // [2 bh, 8] items per XCD
  int32_t* shoff;     // [2 bh, 8] queue offsets
  uint8_t* spx;       // [2 bh, nb] XCD and length class of each position
  int32_t* srng;      // [2 bh, 9] XCD range starts
};
struct TopkArgs {
  const float* scores;
  int32_t *row_ptr, *col_idx, *col_ptr, *row_idx;
  int bh, nb;
  int64_t k;
  TopkWs ws;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
// Per-row TopK (the VSA router baseline): every row keeps its own k / nb largest
// scores, CSR then CSC (uses ws.colcnt and ws.bitmap)
hipError_t launch_topk_rows(const TopkArgs& a, hipStream_t st);
// CSC from a caller CSR (uses ws.colcnt and ws.bitmap)
hipError_t launch_plan(const TopkArgs& a, hipStream_t st);

// Work schedule of the fine branch (sched.hip), built from the CSR and the
// CSC.  Per side (query cubes for the forward and dQ, KV cubes for dK/dV):
// hdr[16] = {start of queue x in items (x < 8), length of queue x}, then
// items[bh * n], item = bh * n + cube.  Workgroup b of a scheduled kernel
// takes items from queue b mod 8 through the counter ctr[b mod 8] (zeroed
// before the launch), then from the other queues.
constexpr int SCHED_MAXN = 46340;  // cubes per (batch, head) the API admits
struct SchedArgs {
  const int32_t *row_ptr, *col_idx, *col_ptr, *row_idx;
  int32_t *row_hdr, *row_items, *col_hdr, *col_items;
  // workspace, for the query side's lists then the KV side's (2 bh entries)
  uint32_t* keys;             // [2 bh, n]
  int32_t *order, *tmp;       // [2 bh, n]
  int32_t *cnt, *hoff;        // [2 bh, 8]
  uint8_t* px;                // [2 bh, n]: XCD << 5 | length class of each position
  int32_t* rng;               // [2 bh, 9]: XCD range starts
  int bh, n;
  int64_t kph;
  int ntc;                    // text cubes: items n .. n + ntc - 1 of every (batch, head), ahead of its range
};
hipError_t launch_sched(const SchedArgs& a, hipStream_t st);

struct AttnArgs {
  const void *q, *k, *v;
  const int32_t *row_ptr, *col_idx;   // CSR (ignored when dense)
  void* o;                            // storage dtype (fine) or fp32 (dense)
  float* lse;                         // [bh, out_rows] natural log
  int bh;
  int nq;                             // query cubes per (batch, head)
  int nkv;                            // kv cubes per (batch, head) (dense)
  int seq;                            // valid tokens per head (rows >= seq are padding)
  int ld;                             // token rows per head in q/k/v buffers
  int out_rows;                       // token rows per head in o / lse
  int64_t kph;                        // col_idx entries per (batch, head)
  int d;
  bool bf16, dense;
  float scale_log2;
  int ct, cy, cx;                     // cube grid for the blocked visiting order (0 = linear)
  PadGrid pad;                        // fine branch on a padded grid: pad keys masked, pad rows zero
  int bs;                             // fine: 2^bs cubes per block; the CSR lists blocks (nq, nkv count cubes)
  int ntc, ntext;                     // fine: text cubes after the nq video cubes, and their tokens (0 = none)
  const int32_t *sq_hdr, *sq_items;   // fine: the schedule's query-cube queues (NULL: one workgroup per cube)
  int32_t* sq_ctr;                    //   their 8 counters (workspace)
};
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t st);

struct AttnBwdArgs {
  const void *q, *k, *v, *o, *d_o;
  const float* lse;                   // [bh, ld] natural log (fine branch)
  const float* stats;                 // dense: [bh, ld] pairs (lse * log2 e, -rowsum(dO * O)); +inf lse = masked row
  float* stats_out;                   // fine: workspace for the same pairs, written by the dQ kernel
  const int32_t *row_ptr, *col_idx, *col_ptr, *row_idx;
  const float *dq_add, *dk_add, *dv_add;  // [bh, nkv >> bs, d] per-block terms added as row/n, n real tokens (or NULL)
  void *dq, *dk, *dv;                 // storage dtype (fine) or fp32 (dense)
  int bh, nq, nkv, seq, ld, out_rows;
  int64_t kph;
  int d;
  bool bf16, dense;
  float scale;
  float scale_log2;
  int ct, cy, cx;                     // cube grid for the blocked visiting order (0 = linear)
  PadGrid pad;                        // fine branch on a padded grid (per-block terms added as row/n, n real tokens)
  int bs;                             // fine: 2^bs cubes per block; CSR / CSC and the per-block terms are per block
  int ntc, ntext;                     // fine: text cubes after the nq video cubes, and their tokens (0 = none)
  const int32_t *sq_hdr, *sq_items;   // fine: the schedule's query-cube queues (NULL: one workgroup per cube)
  const int32_t *sk_hdr, *sk_items;   //   and KV-cube queues
  int32_t* sq_ctr;                    //   8 counters for the dQ pass and 8 for the dK/dV pass (workspace)
};
hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t st);

struct GateArgs {
  const void* x;          // [batch, L, dm]
  const float* w_g;       // [dm, heads]
  void* wt;               // workspace: gate weights repacked for the MFMA operands
  const float* oc_hat;    // [bh, nb, d] fp32
  const void* o_f;
  void* o;
  float* g;               // [bh, L]
  int batch, heads, nb, d, dm;   // nb cubes
  bool bf16;
  PadGrid pad;            // pad rows: g = 0, O = 0
  int bs;                 // 2^bs cubes per coarse token: O_hat_c row of cube c is c >> bs
  int ld;                 // token rows per head in o_f / o (video slots, then text rows, copied O = O_f)
};
hipError_t launch_gate_fwd(const GateArgs& a, hipStream_t st);

// tokens per dW_g partial sum of the gate backward (the partials are then
// reduced in a fixed order, so dW_g does not depend on the launch)
constexpr int DW_TC = 2048;

struct GateBwdArgs {
  const void* x;
  const float* w_g;
  void* wt;               // workspace repack (as forward)
  const float* oc_hat;    // [bh, nb, d]
  const float* g;         // [bh, L]
  const void* d_o;        // [bh, L, d]
  float* dpre;            // workspace [bh, L]
  void* doc;              // workspace [bh, nbp, d] storage dtype: dO_hat_c
  const float* lse_c;     // [bh, nb] natural log, from the forward
  float* stats_c;         // workspace [bh, nbp] pairs (lse_c * log2 e, -rowsum(dO_hat_c * O_hat_c)); pad rows (+inf, 0)
  float* dw_part;         // workspace [nchunk, dm, heads]
  void* dx;
  float* dw_g;
  int batch, heads, nb, nbp, d, dm, nchunk;   // nb cubes; nbp coarse rows (blocks rounded up to 64)
  bool bf16;
  PadGrid pad;            // pad rows: dpre = 0 (so dX = 0 and X there adds nothing to dW_g)
  int bs;                 // 2^bs cubes per coarse token
  float* doc_part;        // workspace [bh, nb, d] fp32 when bs > 0: per-cube sums of dO_hat_c, added in pairs
  int ld;                 // token rows per head in d_o (video slots, then text rows)
};
hipError_t launch_gate_bwd(const GateBwdArgs& a, hipStream_t st);

hipError_t launch_fill_u32(uint32_t* p, uint32_t val, size_t n, hipStream_t st);

// Grid of a scheduled kernel: the workgroups of `threads` threads that fit on
// the current device at once (multiprocessors x resident blocks of fn), a
// multiple of 8 so every XCD gets the same number, at most `items` rounded up
// to 8 and at least 8.
int resident_grid(const void* fn, int threads, int items);

// Diagnostic timer hooks (api.hip): bracket one launch of kernel `kid`.
enum TimerKernel { TK_FINE_FWD = 0, TK_BWD_DKDV = 1, TK_BWD_DQ = 2, TK_ROUTER_LSE = 3, TK_ROUTER_SCORES = 4 };
void timer_before(int kid, hipStream_t st);
void timer_after(int kid, hipStream_t st);

}  // namespace vsa2
