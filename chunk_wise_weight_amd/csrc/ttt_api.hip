// C ABI of the chunk-wise fast-weight library: handle, argument checks, the
// token layout of a call, scratch management and the launch sequence.
//
// One call of ttt_forward_chunked runs, on the caller's stream:
//   1. target gather      V^T = eta * E_tgt[ids shifted by one]^T (next-token target,
//                         eta folded in), or the general target Conv1D(X0) W_target:
//                         tap sums of the token embeddings, then one GEMM into V^T
//   2. up/gate GEMM       Z = SiLU(x W_gate^T) * (x W_up^T) (and, on the fp32 path, Z^T)
//   2b. optional clipping per-chunk factors c_i = min(1, tau/||eta V_i^T Z_i||_F)
//                         from chunk Grams; V^T's rows of chunk i scaled by c_i
//   3. state update       D += rank-C updates eta V_i^T Z_i over the whole
//                         block, the fp32 state resident in registers; a
//                         snapshot of W_down0 + D at the start of every group of G chunks
//   4. group scores       P = Z Z^T masked to earlier chunks of the group
//   5. output GEMM        y = Z snapshot^T + P V
//   6. optional W_final = W_down0 + D (the handle keeps each sequence's state as
//                         D, the change since its last reset)
// Steps 3-5 are the exclusive prefix over chunk updates (iplexlaw.co.kr sec. 6;
// paperlayer.ai App. B) taken at two levels: across groups through the
// snapshots, inside a group through the block-causal term. The result equals
// the sequential apply-then-update loop up to rounding.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/ttt.h"
#include "launch.h"

namespace {

thread_local std::string g_err;

int fail(int code, const std::string &msg) {
  g_err = msg;
  return code;
}

#define HIP_TRY(expr)                                                                          \
  do {                                                                                         \
    hipError_t _e = (expr);                                                                    \
    if (_e != hipSuccess) return fail(TTT_E_HIP, std::string(#expr) + ": " + hipGetErrorString(_e)); \
  } while (0)

constexpr int kMaxDim = 65536;
constexpr int kMaxBatch = 4096;
constexpr int kMaxT = 1 << 23;
constexpr int kDefaultGroupTokens = 1024;
// group starts fall on the update kernel's 32-token stage boundaries
constexpr int kGroupAlign = 64;  // a group starts on a 64-token block of the K-blocked V^T
// profiled phases: gather, up/gate, clip factors, update, scores, output, final copy
constexpr int kPhases = 7;
// event sets kept for ttt_phase_times: one per launch sequence (a forward call, or one document of it)
constexpr int kEvRing = 16;
constexpr int kMaxTaps = 64;

int gcd_int(int a, int b) {
  while (b) {
    int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

struct Plan {
  int C;        // chunk length used for the call (C, or T when C >= T)
  int G;        // chunks per group
  int L;        // tokens per group
  int ngroups;  // groups in the call
  int T_pad;    // slots per sequence in scratch
  int intra;    // a group holds more than one chunk
};

int make_plan(int T, int C, int G_override, Plan &p) {
  if (T < 0 || T > kMaxT) return fail(TTT_E_SHAPE, "T out of range [0, 2^23]");
  if (C < 1) return fail(TTT_E_SHAPE, "chunk length C must be >= 1");
  if (G_override < 0) return fail(TTT_E_SHAPE, "group size G must be >= 0");
  p.T_pad = (int)round_up_ll(T, 256);
  if (T == 0) {
    p.C = C;
    p.G = 1;
    p.L = 8;
    p.ngroups = 0;
    p.intra = 0;
    return TTT_OK;
  }
  const int Ce = C < T ? C : T;
  if (Ce == T) {  // a single chunk: one group, no within-group term
    p.C = T;
    p.G = 1;
    p.L = (int)round_up_ll(T, 8);
    p.ngroups = 1;
    p.intra = 0;
    return TTT_OK;
  }
  const int step = kGroupAlign / gcd_int(Ce, kGroupAlign);
  long long G;
  if (G_override > 0) {
    if (((long long)G_override * Ce) % kGroupAlign != 0)
      return fail(TTT_E_SHAPE, "G*C must be a multiple of 64 (G=" + std::to_string(G_override) +
                                   ", C=" + std::to_string(Ce) + ")");
    G = G_override;
  } else {
    G = (kDefaultGroupTokens + Ce / 2) / Ce;
    if (G < 1) G = 1;
    G = round_up_ll(G, step);
  }
  const long long L = G * Ce;
  p.C = Ce;
  p.G = (int)(G < (1 << 30) ? G : (1 << 30));
  if (L >= T) {  // one group; its length only needs to cover T
    p.L = (int)round_up_ll(T, 8);
    p.ngroups = 1;
  } else {
    p.L = (int)L;
    p.ngroups = (int)((T + L - 1) / L);
  }
  p.intra = G > 1 ? 1 : 0;
  return TTT_OK;
}

// Workspace of ttt_forward_chunked_noalloc: a file-scope device array, so that
// entry point never allocates. Every GPU the library runs on holds its own
// copy, at its own address, until the process ends. In host code the name is
// only a stand-in: the device address comes from hipGetSymbolAddress, taken
// once per device with that device current (in ttt_init) and kept in
// g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = TTT_NOALLOC_WORKSPACE_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The device address of this device's `scratch` (dev current). Taken once per device.
int scratch_ptr_for(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(TTT_E_NODEV, "device index beyond the library's table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(TTT_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return TTT_OK;
}

}  // namespace

struct ttt_handle {
  int d = 0, f = 0, C = 0, max_batch = 0, G_override = 0, device = 0;
  float eta = 0.f;
  float clip_tau = 0.f;     // > 0: Frobenius clipping of each chunk update
  int conv_K = 0;           // > 0: general target with K taps
  int y_f32 = 0;            // bf16 handle: y written as fp32
  int cus = 256;            // compute units of the device
  void *pin = nullptr;      // pinned host staging of the packed-documents tables
  size_t pin_bytes = 0;
  hipEvent_t pin_ev = nullptr;  // recorded after the last copy out of `pin`
  bool pin_used = false;
  float *conv_w = nullptr;  // [K][d] fp32 tap weights
  void *Wt = nullptr;       // bf16: W_target^T [d][d]; f32: W_target [d][d]
  ttt_dtype dt = TTT_BF16;
  void *Wug = nullptr;      // bf16: [d/64][2f][64] (rows interleaved); f32: [2][f][d]
  float *W0 = nullptr;      // [d][f] fp32 image of W_down0
  void *W0p = nullptr;      // bf16: W_down0 as planes [f/8][d][8] (the snapshot layout)
  float *state = nullptr;   // [max_batch][d][f]: D = W - W_down0, the change since the last reset
  void *ws = nullptr;       // scratch
  size_t ws_bytes = 0;
  size_t fixed_bytes = 0;
  bool profiling = false, events_made = false, timed = false;
  hipEvent_t ev[kEvRing][kPhases + 1] = {};
  int ev_next = 0;        // the ring slot the next launch sequence records into
  int ev_pending = 0;     // launch sequences recorded since the last ttt_phase_times, still in the ring
  int calls_pending = 0;  // public forward calls since the last ttt_phase_times
  double ev_fold[kPhases] = {};  // phase sums of the sets folded out of the ring since the last read
  float ev_mean[kPhases] = {};
};

namespace {

int check_device(int *dev_out) {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return fail(TTT_E_NODEV, "no HIP device visible");
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  HIP_TRY(hipGetDeviceProperties(&prop, dev));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(TTT_E_NODEV, std::string("device is ") + prop.gcnArchName + ", this library runs on gfx950 only");
  *dev_out = dev;
  return TTT_OK;
}

void free_handle(ttt_handle *h) {
  if (!h) return;
  (void)hipDeviceSynchronize();
  if (h->Wug) (void)hipFree(h->Wug);
  if (h->W0) (void)hipFree(h->W0);
  if (h->W0p) (void)hipFree(h->W0p);
  if (h->state) (void)hipFree(h->state);
  if (h->conv_w) (void)hipFree(h->conv_w);
  if (h->Wt) (void)hipFree(h->Wt);
  if (h->ws) (void)hipFree(h->ws);
  if (h->pin) (void)hipHostFree(h->pin);
  if (h->pin_ev) (void)hipEventDestroy(h->pin_ev);
  if (h->events_made)
    for (auto &set : h->ev)
      for (auto &e : set) (void)hipEventDestroy(e);
  delete h;
}

struct Scratch {
  void *VT, *Z, *ZT, *snap, *P, *Vrow, *rowpart, *cfac, *U, *gv, *tabs, *state_tmp;
  size_t total;
};

// Kernels move 16-byte vectors: device pointers handed in must be 16-byte aligned.
bool misaligned(const void *p) { return ((uintptr_t)p & 15) != 0; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Scratch of one call over S slots and G snapshot groups of L tokens (lay), for B caller sequences.
// tab_bytes: the packed-documents tables (0 otherwise), followed by B fp32 states for their final values.
Scratch scratch_layout(const ttt_handle *h, const Layout &lay, bool need_zt, bool need_p, bool clip,
                       bool need_vrow, int wspan, bool conv, size_t tab_bytes) {
  const size_t es = h->dt == TTT_BF16 ? 2 : 4;
  const size_t S = (size_t)lay.n_slots(), G = (size_t)lay.n_groups();
  const size_t vt = align256(es * S * h->d);
  const size_t z = align256(es * S * h->f);
  const size_t zt = need_zt ? z : 0;
  const size_t sn = align256(es * G * h->d * h->f);
  const size_t pp = need_p ? align256(es * G * lay.L * lay.L) : 0;
  const size_t vr = need_vrow ? align256(es * S * h->d) : 0;
  const size_t rp = clip ? align256(4 * S * wspan) : 0;
  const size_t cf = clip ? align256(4 * (size_t)lay.n_seq() * ((lay.T_pad + lay.C - 1) / lay.C)) : 0;
  const size_t uu = conv ? align256(es * S * h->d) : 0;
  const size_t gvb = clip && h->dt == TTT_BF16 ? align256(clip_gram_scratch_bytes(lay, wspan)) : 0;
  const size_t tb = align256(tab_bytes);
  const size_t stt = tab_bytes ? align256((size_t)lay.B * h->d * h->f * 4) : 0;
  Scratch s;
  size_t off = 0;
  auto take = [&](void *&ptr, size_t n) {
    ptr = (void *)off;
    off += n;
  };
  take(s.VT, vt);
  take(s.Z, z);
  take(s.ZT, zt);
  take(s.snap, sn);
  take(s.P, pp);
  take(s.Vrow, vr);
  take(s.rowpart, rp);
  take(s.cfac, cf);
  take(s.U, uu);
  take(s.gv, gvb);
  take(s.tabs, tb);
  take(s.state_tmp, stt);
  s.total = off;
  return s;
}

// Packed documents as sequences of their own (bf16 path): the host tables.
struct DocPlan {
  std::vector<SeqInfo> seqs;
  std::vector<int> tile_seq, group_seq;
  long long S = 0;  // slots
  long long G = 0;  // groups
  size_t bytes() const { return seqs.size() * sizeof(SeqInfo) + (tile_seq.size() + group_seq.size()) * 4; }
};

void *at(void *base, void *off) { return (char *)base + (size_t)off; }

}  // namespace

namespace {

// Adds the phase times of ring slot k (a recorded set) to sum[]; waits for the set to complete.
int add_set_times(ttt_handle *h, int k, double *sum) {
  hipEvent_t *e = h->ev[k];
  HIP_TRY(hipEventSynchronize(e[kPhases]));
  for (int i = 0; i < kPhases; ++i) {
    float t = 0.f;
    HIP_TRY(hipEventElapsedTime(&t, e[i], e[i + 1]));
    sum[i] += t;
  }
  return TTT_OK;
}

// Before a launch sequence records into the ring: when every slot still holds
// a set not yet read, the oldest one (the slot about to be reused) is folded
// into running sums first. This waits for that set, recorded 16 launch
// sequences earlier, to finish.
int ring_make_room(ttt_handle *h) {
  if (h->ev_pending < kEvRing) return TTT_OK;
  const int rc = add_set_times(h, h->ev_next, h->ev_fold);
  if (rc) return rc;
  --h->ev_pending;
  return TTT_OK;
}

// One forward over B sequences of T tokens whose states are state[0 .. B).
// ext_ws: a caller-provided workspace of ext_cap bytes used instead of the
// handle's scratch (NULL: the handle's, grown with hipMalloc when needed).
// dp: packed documents run as sequences of their own (bf16 path, eta != 0;
// also with clipping and the general target), with the plan dpl shared by
// every document.
int forward_impl(ttt_handle *h, const void *x, const int32_t *ids, const void *E_tgt, int vocab, int B, int T,
                 void *y, float *state, float *W_final, hipStream_t s_in, void *ext_ws = nullptr,
                 size_t ext_cap = 0, const DocPlan *dp = nullptr, const Plan *dpl = nullptr) {
  const bool learn = h->eta != 0.f;
  Plan pl;
  int rc = TTT_OK;
  if (dp)
    pl = *dpl;
  else
    rc = make_plan(T, h->C, learn ? h->G_override : 0, pl);
  if (rc) return rc;
  if (!learn && pl.ngroups > 0) {  // no updates: one group, the entry state serves every chunk
    pl.ngroups = 1;
    pl.L = (int)round_up_ll(T, 8);
    pl.intra = 0;
  }
  hipStream_t s = s_in;
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev != h->device) return fail(TTT_E_ARG, "current device differs from the handle's device");
  const size_t df = (size_t)h->d * h->f;
  const bool empty = B == 0 || T == 0;

  const bool clip = learn && h->clip_tau > 0.f;
  Layout lay{B, T, pl.T_pad, pl.C, pl.L, pl.ngroups, h->d, h->f, learn ? pl.intra : 0};
  if (dp) {
    lay.nseq = (int)dp->seqs.size();
    lay.S = (int)dp->S;
    lay.G = (int)dp->G;
    lay.tab = true;  // the table pointers are set to its device copy below
  }
  const int wspan = empty ? 1 : clip_wspan(lay, h->dt == TTT_BF16);
  const bool conv = h->conv_K > 0 && (learn || lay.intra);
  // With clipping on the plain bf16 target, the Gram kernel reads the target
  // rows from E through the ids, and the gather runs after the clipping
  // factors and writes V^T already scaled: no row-major copy of V, no
  // scaling pass.
  const bool gram_e =
      clip && !conv && h->dt == TTT_BF16 && (long long)vocab * h->d * 2 < (1LL << 31);
  // Z^T only on the fp32 path: the bf16 update reads Z's blocks transposed
  Scratch sc = empty ? Scratch{}
                     : scratch_layout(h, lay, learn && h->dt != TTT_BF16, learn && pl.intra, clip, clip && !gram_e,
                                      wspan, conv, dp ? dp->bytes() : 0);
  if (ext_ws && sc.total > ext_cap)
    return fail(TTT_E_SHAPE, "the call needs " + std::to_string(sc.total) + " bytes of workspace, more than the " +
                                 std::to_string(ext_cap) + " available");

  const bool prof = h->profiling;
  if (prof) {
    rc = ring_make_room(h);
    if (rc) return rc;
  }
  hipEvent_t *ev = h->ev[h->ev_next];
  auto close_events = [h]() {
    h->ev_next = (h->ev_next + 1) % kEvRing;
    ++h->ev_pending;
    h->timed = true;
  };
  if (prof) HIP_TRY(hipEventRecord(ev[0], s));
  if (empty) {
    if (prof) {
      for (int i = 1; i <= kPhases; ++i) HIP_TRY(hipEventRecord(ev[i], s));
      close_events();
    }
    if (W_final && B > 0) HIP_TRY(launch_add_state_f32(h->W0, state, W_final, B, (long long)df, s));
    return TTT_OK;
  }

  if (!ext_ws && sc.total > h->ws_bytes) {
    HIP_TRY(hipStreamSynchronize(s));
    HIP_TRY(hipDeviceSynchronize());
    if (h->ws) HIP_TRY(hipFree(h->ws));
    h->ws = nullptr;
    h->ws_bytes = 0;
    if (hipMalloc(&h->ws, sc.total) != hipSuccess) {
      (void)hipGetLastError();
      return fail(TTT_E_NOMEM, "allocating " + std::to_string(sc.total) + " bytes of scratch");
    }
    h->ws_bytes = sc.total;
  }
  void *ws = ext_ws ? ext_ws : h->ws;
  void *VT = at(ws, sc.VT), *Z = at(ws, sc.Z), *ZT = at(ws, sc.ZT), *snap = at(ws, sc.snap), *P = at(ws, sc.P);
  void *Vrow = clip && !gram_e ? at(ws, sc.Vrow) : nullptr;
  float *rowpart = (float *)at(ws, sc.rowpart), *cfac = (float *)at(ws, sc.cfac);
  float *gv = (float *)at(ws, sc.gv);
  void *U = at(ws, sc.U);
  float *state_out = state;
  if (dp) {
    // the tables, through pinned staging (the previous call's copy out of it must have finished)
    const size_t nb = dp->bytes();
    if (h->pin_used) HIP_TRY(hipEventSynchronize(h->pin_ev));
    if (nb > h->pin_bytes) {
      if (h->pin) HIP_TRY(hipHostFree(h->pin));
      h->pin = nullptr;
      h->pin_bytes = 0;
      if (hipHostMalloc(&h->pin, nb) != hipSuccess) {
        (void)hipGetLastError();
        return fail(TTT_E_NOMEM, "allocating pinned staging for the document tables");
      }
      h->pin_bytes = nb;
    }
    if (!h->pin_ev) HIP_TRY(hipEventCreateWithFlags(&h->pin_ev, hipEventDisableTiming));
    char *hp = (char *)h->pin;
    const size_t b0 = dp->seqs.size() * sizeof(SeqInfo), b1 = dp->tile_seq.size() * 4;
    std::memcpy(hp, dp->seqs.data(), b0);
    std::memcpy(hp + b0, dp->tile_seq.data(), b1);
    std::memcpy(hp + b0 + b1, dp->group_seq.data(), dp->group_seq.size() * 4);
    char *dt = (char *)at(ws, sc.tabs);
    HIP_TRY(hipMemcpyAsync(dt, hp, nb, hipMemcpyHostToDevice, s));
    HIP_TRY(hipEventRecord(h->pin_ev, s));
    h->pin_used = true;
    lay.info = reinterpret_cast<const SeqInfo *>(dt);
    lay.tile_seq = reinterpret_cast<const int *>(dt + b0);
    lay.group_seq = reinterpret_cast<const int *>(dt + b0 + b1);
    // final states go to a copy: the first document of a sequence reads the state its last one writes
    state_out = (float *)at(ws, sc.state_tmp);
  }

  if (h->dt == TTT_BF16) {
    if (conv) {
      HIP_TRY(launch_conv_taps_bf16(ids, (const bf16_t *)E_tgt, vocab, h->conv_w, h->conv_K, (bf16_t *)U, lay, s));
      HIP_TRY(launch_target_gemm_bf16((const bf16_t *)U, (const bf16_t *)h->Wt, (bf16_t *)VT, (bf16_t *)Vrow, h->eta,
                                      lay, h->cus, s));
    } else if ((learn || lay.intra) && !gram_e) {
      HIP_TRY(launch_gather_vt_bf16(ids, (const bf16_t *)E_tgt, vocab, (bf16_t *)VT, (bf16_t *)Vrow, nullptr, h->eta,
                                    lay, s));
    }
    if (prof) HIP_TRY(hipEventRecord(ev[1], s));
    HIP_TRY(launch_a1_bf16((const bf16_t *)x, (const bf16_t *)h->Wug, (bf16_t *)Z, lay, s));
    if (prof) HIP_TRY(hipEventRecord(ev[2], s));
    if (clip) {
      HIP_TRY(launch_chunk_gram_bf16((const bf16_t *)Z, (const bf16_t *)Vrow, (const bf16_t *)E_tgt, ids, vocab, gv,
                                     rowpart, wspan, lay, h->cus, s));
      HIP_TRY(launch_chunk_factors(rowpart, cfac, wspan, h->eta, h->clip_tau, lay, s));
      if (gram_e)
        HIP_TRY(launch_gather_vt_bf16(ids, (const bf16_t *)E_tgt, vocab, (bf16_t *)VT, nullptr, cfac, h->eta, lay, s));
      else
        HIP_TRY(launch_scale_vt_bf16((bf16_t *)VT, cfac, lay, s));
    }
    if (prof) HIP_TRY(hipEventRecord(ev[3], s));
    if (learn) {
      HIP_TRY(launch_update_bf16((const bf16_t *)Z, (const bf16_t *)VT, state, state_out, (bf16_t *)snap,
                                 (const bf16_t *)h->W0p, lay, h->cus, s));
      if (state_out != state)
        HIP_TRY(hipMemcpyAsync(state, state_out, (size_t)B * df * 4, hipMemcpyDeviceToDevice, s));
    } else {
      for (int b = 0; b < B; ++b)
        HIP_TRY(launch_state_to_snap_bf16(h->W0, state + (size_t)b * df, (bf16_t *)snap + (size_t)b * df, h->d,
                                          h->f, s));
    }
    if (prof) HIP_TRY(hipEventRecord(ev[4], s));
    if (lay.intra) HIP_TRY(launch_scores_bf16((const bf16_t *)Z, (bf16_t *)P, lay, h->cus, s));
    if (prof) HIP_TRY(hipEventRecord(ev[5], s));
    HIP_TRY(launch_out_bf16((const bf16_t *)Z, (const bf16_t *)P, (const bf16_t *)snap, (const bf16_t *)VT, y,
                            h->y_f32, lay, h->cus, s));
  } else {
    if (conv) {
      HIP_TRY(launch_conv_taps_f32(ids, (const float *)E_tgt, vocab, h->conv_w, h->conv_K, (float *)U, lay, s));
      HIP_TRY(launch_target_gemm_f32((const float *)U, (const float *)h->Wt, (float *)VT, (float *)Vrow, lay, s));
    } else if (learn || lay.intra) {
      HIP_TRY(launch_gather_vt_f32(ids, (const float *)E_tgt, vocab, (float *)VT, (float *)Vrow, lay, s));
    }
    if (prof) HIP_TRY(hipEventRecord(ev[1], s));
    HIP_TRY(launch_a1_f32((const float *)x, (const float *)h->Wug, (float *)Z, (float *)ZT, h->eta, learn ? 1 : 0,
                          lay, s));
    if (prof) HIP_TRY(hipEventRecord(ev[2], s));
    if (clip) {
      HIP_TRY(launch_chunk_gram_f32((const float *)Z, (const float *)Vrow, rowpart, lay, s));
      HIP_TRY(launch_chunk_factors(rowpart, cfac, wspan, h->eta, h->clip_tau, lay, s));
      HIP_TRY(launch_scale_vt_f32((float *)VT, cfac, lay, s));
    }
    if (prof) HIP_TRY(hipEventRecord(ev[3], s));
    if (learn) {
      HIP_TRY(launch_update_f32((const float *)ZT, (const float *)VT, state, (float *)snap, h->W0, lay, s));
    } else {
      HIP_TRY(launch_add_state_f32(h->W0, state, (float *)snap, B, (long long)df, s));
    }
    if (prof) HIP_TRY(hipEventRecord(ev[4], s));
    if (lay.intra) HIP_TRY(launch_scores_f32((const float *)Z, (float *)P, h->eta, lay, s));
    if (prof) HIP_TRY(hipEventRecord(ev[5], s));
    HIP_TRY(launch_out_f32((const float *)Z, (const float *)P, (const float *)snap, (const float *)VT, (float *)y,
                           lay, s));
  }
  if (prof) HIP_TRY(hipEventRecord(ev[6], s));
  if (W_final) HIP_TRY(launch_add_state_f32(h->W0, state, W_final, B, (long long)df, s));
  if (prof) {
    HIP_TRY(hipEventRecord(ev[7], s));
    close_events();
  }
  return TTT_OK;
}


}  // namespace

extern "C" {

const char *ttt_last_error(void) { return g_err.c_str(); }

int ttt_plan(int T, int C, int G_override, int *G, int *L, int *ngroups, int *T_pad) {
  Plan p;
  int rc = make_plan(T, C, G_override, p);
  if (rc) return rc;
  if (G) *G = p.G;
  if (L) *L = p.L;
  if (ngroups) *ngroups = p.ngroups;
  if (T_pad) *T_pad = p.T_pad;
  return TTT_OK;
}

int ttt_init(ttt_handle **out, const void *W_up, const void *W_gate, const void *W_down0, int d, int f, int C,
             float eta, ttt_dtype dt, int max_batch, void *hip_stream) {
  if (!out) return fail(TTT_E_NULL, "out is NULL");
  *out = nullptr;
  if (!W_up || !W_gate || !W_down0) return fail(TTT_E_NULL, "W_up, W_gate and W_down0 must be non-NULL");
  if (misaligned(W_up) || misaligned(W_gate) || misaligned(W_down0))
    return fail(TTT_E_ARG, "W_up, W_gate and W_down0 must be 16-byte aligned");
  if (dt != TTT_F32 && dt != TTT_BF16) return fail(TTT_E_DTYPE, "dtype must be TTT_F32 or TTT_BF16");
  if (d < 64 || f < 64 || d > kMaxDim || f > kMaxDim || d % 64 || f % 64)
    return fail(TTT_E_SHAPE, "d and f must be multiples of 64 in [64, 65536]");
  if (dt == TTT_BF16 && (d % 256 || f % 256))
    return fail(TTT_E_SHAPE, "the bf16 path needs d and f to be multiples of 256");
  if (C < 1) return fail(TTT_E_SHAPE, "chunk length C must be >= 1");
  if (!std::isfinite(eta)) return fail(TTT_E_ARG, "eta must be finite");
  if (max_batch < 1 || max_batch > kMaxBatch) return fail(TTT_E_SHAPE, "max_batch must be in [1, 4096]");
  int dev = 0;
  int rc = check_device(&dev);
  if (rc) return rc;
  void *sp = nullptr;  // set-up of ttt_forward_chunked_noalloc's workspace on this device
  rc = scratch_ptr_for(dev, &sp);
  if (rc) return rc;

  hipStream_t s = (hipStream_t)hip_stream;
  ttt_handle *h = new ttt_handle();
  {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
      h->cus = prop.multiProcessorCount;
  }
  h->d = d;
  h->f = f;
  h->C = C;
  h->eta = eta;
  h->dt = dt;
  h->max_batch = max_batch;
  h->device = dev;
  const size_t es = dt == TTT_BF16 ? 2 : 4;
  const size_t df = (size_t)d * f;
  auto bail = [&](int code, const std::string &m) {
    free_handle(h);
    return fail(code, m);
  };
  if (hipMalloc(&h->Wug, 2 * df * es) != hipSuccess) return bail(TTT_E_NOMEM, "allocating W_up/W_gate copy");
  if (hipMalloc((void **)&h->W0, df * 4) != hipSuccess) return bail(TTT_E_NOMEM, "allocating W_down0 image");
  if (hipMalloc((void **)&h->state, df * 4 * max_batch) != hipSuccess)
    return bail(TTT_E_NOMEM, "allocating fast-weight states");
  if (dt == TTT_BF16 && hipMalloc(&h->W0p, df * 2) != hipSuccess) return bail(TTT_E_NOMEM, "allocating W_down0 planes");
  h->fixed_bytes = 2 * df * es + df * 4 + df * 4 * max_batch + (dt == TTT_BF16 ? df * 2 : 0);
  hipError_t e = hipSuccess;
  if (dt == TTT_BF16) {
    e = launch_interleave_ug_bf16((const bf16_t *)W_up, (const bf16_t *)W_gate, (bf16_t *)h->Wug, f, d, s);
    if (e == hipSuccess) e = launch_bf16_to_f32((const bf16_t *)W_down0, h->W0, (long long)df, s);
    if (e == hipSuccess) e = launch_to_planes_bf16((const bf16_t *)W_down0, (bf16_t *)h->W0p, d, f, s);
  } else {
    e = hipMemcpyAsync(h->Wug, W_up, df * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync((float *)h->Wug + df, W_gate, df * 4, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(h->W0, W_down0, df * 4, hipMemcpyDeviceToDevice, s);
  }
  if (e == hipSuccess) e = launch_fill_f32(h->state, 0.f, (long long)df * max_batch, s);
  if (e != hipSuccess) return bail(TTT_E_HIP, std::string("init copies: ") + hipGetErrorString(e));
  *out = h;
  return TTT_OK;
}

int ttt_set_group_chunks(ttt_handle *h, int G) {
  if (!h) return fail(TTT_E_NULL, "handle is NULL");
  if (G < 0) return fail(TTT_E_SHAPE, "G must be >= 0");
  if (G > 0 && ((long long)G * h->C) % kGroupAlign != 0) return fail(TTT_E_SHAPE, "G*C must be a multiple of 64");
  h->G_override = G;
  return TTT_OK;
}

int ttt_set_clip(ttt_handle *h, float tau) {
  if (!h) return fail(TTT_E_NULL, "handle is NULL");
  if (!(tau >= 0.f)) return fail(TTT_E_ARG, "tau must be >= 0 (0 or +inf: no clipping)");
  h->clip_tau = std::isinf(tau) ? 0.f : tau;
  return TTT_OK;
}

int ttt_set_target_conv(ttt_handle *h, const void *conv_w, int K, const void *W_target, void *hip_stream) {
  if (!h) return fail(TTT_E_NULL, "handle is NULL");
  if (K < 0 || K > kMaxTaps) return fail(TTT_E_ARG, "K must be in [0, 64]");
  hipStream_t s = (hipStream_t)hip_stream;
  if (K == 0) {
    HIP_TRY(hipStreamSynchronize(s));
    if (h->conv_w) HIP_TRY(hipFree(h->conv_w));
    if (h->Wt) HIP_TRY(hipFree(h->Wt));
    h->conv_w = nullptr;
    h->Wt = nullptr;
    h->conv_K = 0;
    return TTT_OK;
  }
  if (!conv_w || !W_target) return fail(TTT_E_NULL, "conv_w and W_target must be non-NULL");
  if (misaligned(conv_w) || misaligned(W_target)) return fail(TTT_E_ARG, "conv_w and W_target must be 16-byte aligned");
  const size_t es = h->dt == TTT_BF16 ? 2 : 4;
  const size_t dd = (size_t)h->d * h->d;
  HIP_TRY(hipStreamSynchronize(s));
  if (h->conv_w) HIP_TRY(hipFree(h->conv_w));
  if (h->Wt) HIP_TRY(hipFree(h->Wt));
  h->conv_w = nullptr;
  h->Wt = nullptr;
  h->conv_K = 0;
  if (hipMalloc((void **)&h->conv_w, (size_t)K * h->d * 4) != hipSuccess ||
      hipMalloc(&h->Wt, dd * es) != hipSuccess) {
    (void)hipGetLastError();
    return fail(TTT_E_NOMEM, "allocating the target convolution weights");
  }
  if (h->dt == TTT_BF16) {
    HIP_TRY(launch_bf16_to_f32((const bf16_t *)conv_w, h->conv_w, (long long)K * h->d, s));
    HIP_TRY(launch_transpose_bf16((const bf16_t *)W_target, (bf16_t *)h->Wt, h->d, s));
  } else {
    HIP_TRY(launch_copy_f32((const float *)conv_w, h->conv_w, (long long)K * h->d, s));
    HIP_TRY(hipMemcpyAsync(h->Wt, W_target, dd * 4, hipMemcpyDeviceToDevice, s));
  }
  h->conv_K = K;
  return TTT_OK;
}

int ttt_set_output_f32(ttt_handle *h, int on) {
  if (!h) return fail(TTT_E_NULL, "handle is NULL");
  h->y_f32 = (on != 0 && h->dt == TTT_BF16) ? 1 : 0;
  return TTT_OK;
}

int ttt_set_profiling(ttt_handle *h, int on) {
  if (!h) return fail(TTT_E_NULL, "handle is NULL");
  if (on && !h->events_made) {
    for (auto &set : h->ev)
      for (auto &e : set) HIP_TRY(hipEventCreate(&e));
    h->events_made = true;
  }
  h->profiling = on != 0;
  h->timed = false;
  h->ev_pending = h->calls_pending = 0;
  for (double &v : h->ev_fold) v = 0.0;
  return TTT_OK;
}

int ttt_phase_times(ttt_handle *h, float *ms, int n) {
  if (!h || !ms) return fail(TTT_E_NULL, "handle or ms is NULL");
  if (n < 0 || n > kPhases) return fail(TTT_E_ARG, "n must be in [0, 7]");
  if (!h->timed) return fail(TTT_E_ARG, "no profiled forward call yet (enable ttt_set_profiling first)");
  if (h->ev_pending > 0 || h->calls_pending > 0) {
    double sum[kPhases];
    for (int i = 0; i < kPhases; ++i) sum[i] = h->ev_fold[i];
    for (int k = 1; k <= h->ev_pending; ++k) {
      const int rc = add_set_times(h, (h->ev_next - k + kEvRing) % kEvRing, sum);
      if (rc) return rc;
    }
    const int calls = h->calls_pending > 0 ? h->calls_pending : 1;
    for (int i = 0; i < kPhases; ++i) h->ev_mean[i] = (float)(sum[i] / calls);
    h->ev_pending = h->calls_pending = 0;
    for (double &v : h->ev_fold) v = 0.0;
  }
  for (int i = 0; i < n; ++i) ms[i] = h->ev_mean[i];
  return TTT_OK;
}

int ttt_workspace_bytes(ttt_handle *h, size_t *bytes) {
  if (!h || !bytes) return fail(TTT_E_NULL, "handle or bytes is NULL");
  *bytes = h->fixed_bytes + h->ws_bytes;
  return TTT_OK;
}

int ttt_reset(ttt_handle *h, int b, void *hip_stream) {
  if (!h) return fail(TTT_E_NULL, "handle is NULL");
  if (b < -1 || b >= h->max_batch) return fail(TTT_E_ARG, "batch index out of range");
  hipStream_t s = (hipStream_t)hip_stream;
  const size_t df = (size_t)h->d * h->f;
  const int lo = b < 0 ? 0 : b, hi = b < 0 ? h->max_batch : b + 1;
  HIP_TRY(launch_fill_f32(h->state + (size_t)lo * df, 0.f, (long long)df * (hi - lo), s));
  return TTT_OK;
}

void ttt_destroy(ttt_handle *h) { free_handle(h); }

int ttt_forward_chunked(ttt_handle *h, const void *x, const int32_t *ids, const void *E_tgt, int vocab, int B, int T,
                        void *y, float *W_final, void *hip_stream) {
  if (!h) return fail(TTT_E_NULL, "handle is NULL");
  if (B < 0 || B > h->max_batch) return fail(TTT_E_SHAPE, "B must be in [0, max_batch]");
  if (T < 0 || T > kMaxT) return fail(TTT_E_SHAPE, "T must be in [0, 2^23]");
  if (B > 0 && T > 0 && (!x || !ids || !E_tgt || !y)) return fail(TTT_E_NULL, "x, ids, E_tgt and y must be non-NULL");
  if (B > 0 && T > 0 && vocab < 1) return fail(TTT_E_SHAPE, "vocab must be >= 1");
  if (B > 0 && T > 0 && (misaligned(x) || misaligned(E_tgt) || misaligned(y)))
    return fail(TTT_E_ARG, "x, E_tgt and y must be 16-byte aligned");
  const int rc = forward_impl(h, x, ids, E_tgt, vocab, B, T, y, h->state, W_final, (hipStream_t)hip_stream);
  if (rc == TTT_OK && h->profiling) ++h->calls_pending;
  return rc;
}

int ttt_forward_chunked_noalloc(ttt_handle *h, const void *x, const int32_t *ids, const void *E_tgt, int vocab,
                                int B, int T, void *y, float *W_final, void *hip_stream) {
  if (!h) return fail(TTT_E_NULL, "handle is NULL");
  if (B < 0 || B > h->max_batch) return fail(TTT_E_SHAPE, "B must be in [0, max_batch]");
  if (T < 0 || T > kMaxT) return fail(TTT_E_SHAPE, "T must be in [0, 2^23]");
  if (B > 0 && T > 0 && (!x || !ids || !E_tgt || !y)) return fail(TTT_E_NULL, "x, ids, E_tgt and y must be non-NULL");
  if (B > 0 && T > 0 && vocab < 1) return fail(TTT_E_SHAPE, "vocab must be >= 1");
  if (B > 0 && T > 0 && (misaligned(x) || misaligned(E_tgt) || misaligned(y)))
    return fail(TTT_E_ARG, "x, E_tgt and y must be 16-byte aligned");
  void *sp = nullptr;
  int rc = scratch_ptr_for(h->device, &sp);  // resolved in ttt_init; a table lookup here
  if (rc) return rc;
  rc = forward_impl(h, x, ids, E_tgt, vocab, B, T, y, h->state, W_final, (hipStream_t)hip_stream, sp,
                    kNoAllocScratchBytes);
  if (rc == TTT_OK && h->profiling) ++h->calls_pending;
  return rc;
}

int ttt_forward_docs(ttt_handle *h, const void *x, const int32_t *ids, const void *E_tgt, int vocab, int B, int T,
                     const int32_t *doc_starts, const int32_t *doc_counts, void *y, float *W_final,
                     void *hip_stream) {
  if (!h) return fail(TTT_E_NULL, "handle is NULL");
  if (B < 0 || B > h->max_batch) return fail(TTT_E_SHAPE, "B must be in [0, max_batch]");
  if (T < 0 || T > kMaxT) return fail(TTT_E_SHAPE, "T must be in [0, 2^23]");
  if (B > 0 && T > 0 && (!x || !ids || !E_tgt || !y)) return fail(TTT_E_NULL, "x, ids, E_tgt and y must be non-NULL");
  if (B > 0 && T > 0 && vocab < 1) return fail(TTT_E_SHAPE, "vocab must be >= 1");
  if (B > 0 && T > 0 && (misaligned(x) || misaligned(E_tgt) || misaligned(y)))
    return fail(TTT_E_ARG, "x, E_tgt and y must be 16-byte aligned");
  if (B > 0 && T > 0 && !doc_counts) return fail(TTT_E_NULL, "doc_counts must be non-NULL");
  long long total = 0;
  for (int b = 0; b < B && T > 0; ++b) {
    if (doc_counts[b] < 0 || doc_counts[b] >= T) return fail(TTT_E_ARG, "doc_counts[b] must be in [0, T)");
    total += doc_counts[b];
  }
  if (total > 0 && !doc_starts) return fail(TTT_E_NULL, "doc_starts must be non-NULL");
  for (int b = 0, k = 0; b < B && T > 0; ++b) {
    int prev = 0;
    for (int j = 0; j < doc_counts[b]; ++j, ++k) {
      if (doc_starts[k] <= prev || doc_starts[k] >= T)
        return fail(TTT_E_ARG, "document starts must increase strictly inside (0, T)");
      prev = doc_starts[k];
    }
  }
  hipStream_t s = (hipStream_t)hip_stream;
  if (B == 0 || T == 0 || total == 0) {
    const int rc = forward_impl(h, x, ids, E_tgt, vocab, B, T, y, h->state, W_final, s);
    if (rc == TTT_OK && h->profiling) ++h->calls_pending;
    return rc;
  }
  const size_t es = h->dt == TTT_BF16 ? 2 : 4;
  const size_t ys = h->dt == TTT_BF16 && !h->y_f32 ? 2 : 4;  // bytes per element of y
  const size_t df = (size_t)h->d * h->f;
  if (h->dt == TTT_BF16 && h->eta != 0.f) {
    // One launch sequence: every document is a sequence of its own in the scan kernels, with its own
    // scratch slots (padded to 256) and snapshot groups; the first document of sequence b continues
    // its state, every later one starts from W_down0, and the last one's final state is kept. Chunks
    // and groups count from each document's first token. One plan serves every document: that of
    // the longest one (a shorter document just has fewer groups).
    DocPlan dp;
    int maxlen = 0;
    for (int b = 0, k = 0; b < B; ++b) {
      int s0 = 0;
      for (int j = 0; j <= doc_counts[b]; ++j) {
        const int s1 = j < doc_counts[b] ? doc_starts[k + j] : T;
        maxlen = s1 - s0 > maxlen ? s1 - s0 : maxlen;
        s0 = s1;
      }
      k += doc_counts[b];
    }
    Plan pl;
    int rc = make_plan(maxlen, h->C, h->G_override, pl);
    if (rc) return rc;
    for (int b = 0, k = 0; b < B; ++b) {
      int s0 = 0;
      for (int j = 0; j <= doc_counts[b]; ++j) {
        const int s1 = j < doc_counts[b] ? doc_starts[k + j] : T;
        const int len = s1 - s0;
        SeqInfo si;
        si.xrow0 = (long long)b * T + s0;
        si.id0 = (long long)b * (T + 1) + s0;
        si.slot0 = (int)dp.S;
        si.len = len;
        si.grp0 = (int)dp.G;
        si.state_in = j == 0 ? b : -1;
        si.state_out = j == doc_counts[b] ? b : -1;
        si.pad_ = 0;
        const int seq = (int)dp.seqs.size();
        dp.seqs.push_back(si);
        const long long tp = round_up_ll(len, 256), ng = len > pl.L ? (len + pl.L - 1) / pl.L : 1;
        for (long long t = 0; t < tp / 256; ++t) dp.tile_seq.push_back(seq);
        for (long long g = 0; g < ng; ++g) dp.group_seq.push_back(seq);
        dp.S += tp;
        dp.G += ng;
        s0 = s1;
      }
      k += doc_counts[b];
    }
    if (dp.S < (1LL << 30) && dp.G < (1LL << 30)) {
      rc = forward_impl(h, x, ids, E_tgt, vocab, B, T, y, h->state, W_final, s, nullptr, 0, &dp, &pl);
      if (rc == TTT_OK && h->profiling) ++h->calls_pending;
      return rc;
    }
  }
  // Otherwise (fp32 handle, or eta = 0): each document runs on its own slice: the state of sequence b returns to
  // W_down0 at every document start, and chunking restarts there. The ids
  // slice keeps the next document's first token as its look-ahead; that
  // target only enters the document's last chunk update, which the reset
  // discards.
  for (int b = 0, k = 0; b < B; ++b) {
    int s0 = 0;
    for (int j = 0; j <= doc_counts[b]; ++j) {
      const int s1 = j < doc_counts[b] ? doc_starts[k + j] : T;
      if (j > 0) HIP_TRY(launch_fill_f32(h->state + (size_t)b * df, 0.f, (long long)df, s));
      const size_t row = ((size_t)b * T + s0) * h->d;
      const int rc = forward_impl(h, (const char *)x + row * es, ids + (size_t)b * (T + 1) + s0, E_tgt, vocab, 1,
                                  s1 - s0, (char *)y + row * ys, h->state + (size_t)b * df, nullptr, s);
      if (rc) return rc;
      s0 = s1;
    }
    k += doc_counts[b];
  }
  if (W_final) HIP_TRY(launch_add_state_f32(h->W0, h->state, W_final, B, (long long)df, s));
  if (h->profiling) ++h->calls_pending;
  return TTT_OK;
}

int ttt_state_delta(ttt_handle *h, float *dW, int B, void *hip_stream) {
  if (!h) return fail(TTT_E_NULL, "handle is NULL");
  if (B < 0 || B > h->max_batch) return fail(TTT_E_SHAPE, "B must be in [0, max_batch]");
  if (B > 0 && !dW) return fail(TTT_E_NULL, "dW must be non-NULL");
  if (B > 0 && misaligned(dW)) return fail(TTT_E_ARG, "dW must be 16-byte aligned");
  const size_t df = (size_t)h->d * h->f;
  if (B > 0)
    HIP_TRY(hipMemcpyAsync(dW, h->state, (size_t)B * df * 4, hipMemcpyDeviceToDevice, (hipStream_t)hip_stream));
  return TTT_OK;
}

}  // extern "C"
