// api.hip -- extern "C" entry points of libtess.so (declared in include/tess.h) and the
// velocity-Verlet kernels of tess_md_steps.
#include <cmath>
#include <cstring>

#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "tess_common.h"

namespace tess {

// ---- optional per-kernel timing --------------------------------------------------------
namespace {
struct TimingState {
  std::mutex mu;
  bool on = false;
  std::map<std::string, std::vector<std::pair<hipEvent_t, hipEvent_t>>> ev;
  std::map<std::string, hipEvent_t> open;
  std::string only;  // when not empty, only this kernel is timed
};
TimingState& timing() {
  static TimingState t;
  return t;
}
}  // namespace

bool timing_on() { return timing().on; }

namespace {
std::atomic<int> g_curve{0};
}
int sort_curve() { return g_curve.load(); }

bool timing_wants(const char* name) {
  TimingState& t = timing();
  if (!t.on) return false;
  std::lock_guard<std::mutex> g(t.mu);
  return t.only.empty() || t.only == name;
}

void timing_mark(const char* name, hipStream_t st, bool begin) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  hipEvent_t e;
  if (hipEventCreate(&e) != hipSuccess) return;
  (void)hipEventRecord(e, st);
  if (begin) {
    t.open[name] = e;
  } else {
    auto it = t.open.find(name);
    if (it == t.open.end()) { (void)hipEventDestroy(e); return; }
    t.ev[name].push_back({it->second, e});
    t.open.erase(it);
  }
}

namespace {

// 16-byte loads read the weights and the workspace
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

constexpr float kAccelConv = 9.648533e-3f;  // eV/A/amu -> A/fs^2

// First half of a velocity-Verlet step: v += dt/2 F/m; x += dt v; flag |x - x_ref| > skin/2.
// Species index of mass_by_species, clamped to [0, S) (an out-of-range species is reported
// by the energy pass through the status word; the clamp keeps every access in bounds).
__device__ __forceinline__ int32_t mass_index(int32_t s, int32_t S) { return min(max(s, 0), S - 1); }

__global__ void k_vv_kick_drift(int32_t n, float dt, const float* __restrict__ F,
                                const int32_t* __restrict__ species,
                                const float* __restrict__ mass, int32_t S,
                                float* __restrict__ pos, float* __restrict__ vel,
                                const float* __restrict__ ref, float half_skin2,
                                int32_t* __restrict__ flag) {
  int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float im = kAccelConv / mass[mass_index(species[i], S)];
  float d2 = 0.0f;
#pragma unroll
  for (int a = 0; a < 3; a++) {
    float v = vel[3 * i + a] + 0.5f * dt * F[3 * i + a] * im;
    float x = pos[3 * i + a] + dt * v;
    vel[3 * i + a] = v;
    pos[3 * i + a] = x;
    float d = x - ref[3 * i + a];
    d2 += d * d;
  }
  if (d2 > half_skin2) atomicOr(flag, 1);
}

// Second half: v += dt/2 F/m.
__global__ void k_vv_kick(int32_t n, float dt, const float* __restrict__ F,
                          const int32_t* __restrict__ species, const float* __restrict__ mass,
                          int32_t S, float* __restrict__ vel) {
  int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float im = kAccelConv / mass[mass_index(species[i], S)];
#pragma unroll
  for (int a = 0; a < 3; a++) vel[3 * i + a] += 0.5f * dt * F[3 * i + a] * im;
}

// Sum over the 256 threads of a block in a fixed order (every thread gets the same value).
__device__ __forceinline__ double block_sum_256(double v) {
  __shared__ double red[4];
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Second half with the block's kinetic-energy sum: v += dt/2 F/m (as k_vv_kick), then
// part[block] = sum of m |v|^2 over the block's atoms in fp64 (amu A^2/fs^2).
__global__ void __launch_bounds__(256) k_vv_kick_ke(int32_t n, float dt,
                                                    const float* __restrict__ F,
                                                    const int32_t* __restrict__ species,
                                                    const float* __restrict__ mass, int32_t S,
                                                    float* __restrict__ vel,
                                                    double* __restrict__ part) {
  int32_t i = blockIdx.x * 256 + threadIdx.x;
  double mv2 = 0.0;
  if (i < n) {
    const float m = mass[mass_index(species[i], S)];
    const float im = kAccelConv / m;
    double v2 = 0.0;
#pragma unroll
    for (int a = 0; a < 3; a++) {
      const float v = vel[3 * i + a] + 0.5f * dt * F[3 * i + a] * im;
      vel[3 * i + a] = v;
      v2 += (double)v * (double)v;
    }
    mv2 = (double)m * v2;
  }
  mv2 = block_sum_256(mv2);
  if (threadIdx.x == 0) part[blockIdx.x] = mv2;
}

constexpr double kAccelConvD = 9.648533e-3;  // eV/A/amu -> A/fs^2, so amu A^2/fs^2 -> eV is 1/it
constexpr double kBoltzmannEv = 8.617333262e-5;  // eV/K

// End of a step with a thermostat or monitors. Every block sums the kinetic-energy block
// sums in the same order, so all blocks obtain the same KE and lambda. Berendsen weak
// coupling: lambda^2 = 1 + (dt/tau)(T0/T - 1) with T = 2 KE / (3 N k_B) (lambda = 1 when
// T = 0); velocities are scaled by lambda. Block 0 writes the traces: KE after scaling
// (lambda^2 KE) and the shortest pair distance, whose squared value it then resets to +inf
// for the next step.
__global__ void __launch_bounds__(256) k_md_thermo(int32_t n, int32_t nparts,
                                                   const double* __restrict__ part,
                                                   int32_t berendsen, double dt_over_tau,
                                                   double t_target, float* __restrict__ vel,
                                                   double* __restrict__ ke_out,
                                                   uint32_t* __restrict__ rmin2_bits,
                                                   float* __restrict__ rmin_out) {
  double s = 0.0;
  for (int32_t k = threadIdx.x; k < nparts; k += 256) s += part[k];
  s = block_sum_256(s);
  const double ke = 0.5 * s / kAccelConvD;
  double lam2 = 1.0;
  if (berendsen) {
    const double T = 2.0 * ke / (3.0 * (double)n * kBoltzmannEv);
    if (T > 0.0) lam2 = 1.0 + dt_over_tau * (t_target / T - 1.0);
    const float lam = (float)sqrt(lam2);
    const int32_t i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
#pragma unroll
      for (int a = 0; a < 3; a++) vel[3 * i + a] *= lam;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (ke_out) *ke_out = lam2 * ke;
    if (rmin_out) {
      *rmin_out = sqrtf(__uint_as_float(*rmin2_bits));
      *rmin2_bits = 0x7f800000u;
    }
  }
}

__global__ void k_set_u32(uint32_t* __restrict__ p, uint32_t v) { *p = v; }
__global__ void k_zero_f64(double* __restrict__ p) { *p = 0.0; }

// After a replayed interval: the traces of its k steps, written by the graph into the
// workspace's staging arrays, are copied to the caller's trace arrays (NULL: not requested).
__global__ void k_copy_traces(int32_t k, const double* __restrict__ ep_in,
                              double* __restrict__ ep_out, const double* __restrict__ ke_in,
                              double* __restrict__ ke_out, const float* __restrict__ rm_in,
                              float* __restrict__ rm_out) {
  const int32_t j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= k) return;
  if (ep_out) ep_out[j] = ep_in[j];
  if (ke_out) ke_out[j] = ke_in[j];
  if (rm_out) rm_out[j] = rm_in[j];
}

inline int32_t gridn(int64_t n, int b) { return (int32_t)((n + b - 1) / b); }

// Steps per interval whose traces a replayed graph stages in the workspace (longer
// intervals run eagerly).
constexpr int32_t kTraceStage = 256;

struct Layout {
  int32_t* status;  // device status word (first word of the workspace)
  NbrWS nbr;
  char* ef;
  int64_t ef_bytes;
  // tess_md_steps scratch
  float* ref_pos;
  int32_t* perm;
  int32_t* flag;    // skin flag: the word after the status word (both read with one copy)
  double* epot;
  double* ke_part;      // kinetic-energy sums, one per block of 256 atoms
  uint32_t* rmin2_bits;  // shortest squared pair distance of the step (float bits)
  double *epot_stage, *ke_stage;  // per-step traces of a replayed interval
  float* rmin_stage;
  int64_t total;
};

Layout layout(char* base, const tess_model_desc* md, int32_t n, int64_t cap) {
  Layout L{};
  Carver cv{base, 0};
  L.status = cv.take<int32_t>(64);
  L.nbr = carve_nbr(cv, n);
  int64_t nn = n > 0 ? n : 1;
  L.ref_pos = cv.take<float>(3 * nn);
  L.perm = cv.take<int32_t>(nn);
  L.flag = L.status + 1;
  L.epot = cv.take<double>(4);
  L.ke_part = cv.take<double>(gridn(nn, 256));
  L.rmin2_bits = cv.take<uint32_t>(64);
  L.epot_stage = cv.take<double>(kTraceStage);
  L.ke_stage = cv.take<double>(kTraceStage);
  L.rmin_stage = cv.take<float>(kTraceStage);
  if (md) {
    L.ef_bytes = ef_workspace_bytes(*md, n, cap);
    L.ef = cv.take<char>(L.ef_bytes);
  }
  L.total = cv.off + 256;
  return L;
}

bool box_ok(const float box[3], float r_cut, float skin) {
  double rcs = (double)r_cut + (double)skin;
  for (int a = 0; a < 3; a++)
    if (!((double)box[a] > 2.0 * rcs) || !std::isfinite(box[a])) return false;
  return true;
}

// ---- neighbour build without allocation (tess_build_neighbors_static) --------------------
// A file-scope device array holds that entry point's scratch (the wrap/sort/cell arrays of the
// rebuild and the status word), so its callers pass no workspace. Each GPU the library runs
// on holds one copy until the process ends. Host code never uses the array's name as an
// address: the device address of each GPU's copy comes from hipGetSymbolAddress, taken once
// per device with that device current.
constexpr int64_t kStaticScratchBytes = int64_t(48) << 20;  // 48 MiB
constexpr int32_t kStaticMaxAtoms = 1 << 19;                // 524,288 atoms
static __device__ __align__(256) char scratch[kStaticScratchBytes];

// Device address of this device's scratch copy (nullptr if it cannot be resolved).
char* static_scratch() {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static char* addr[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = static_cast<char*>(p);
  }
  return addr[dev];
}

__global__ void k_zero_i32(int32_t* __restrict__ p) { *p = 0; }

}  // namespace
}  // namespace tess

using namespace tess;

// ---- graph replay of a rebuild interval (TESS_MD_GRAPH) ----------------------------------
// The k velocity-Verlet steps between two rebuilds are captured once into a HIP graph and
// replayed for every later interval with the same arguments. The key holds everything the
// captured launches bake in: device pointers, sizes, the step count, the time step, the box,
// the model, the skin threshold and the thermostat; the per-step traces are written by the
// graph into fixed staging arrays of the workspace (copied out after each replay), so the
// trace pointers of an interval are not part of the key. One cached graph per process; a
// different key re-captures it.
namespace {
struct GraphKey {
  const void* p[10];
  int64_t i[10];
  float f[8];
  bool operator==(const GraphKey& o) const { return std::memcmp(this, &o, sizeof(*this)) == 0; }
};
struct GraphCache {
  std::mutex mu;
  bool valid = false;
  GraphKey key;
  hipGraphExec_t exec = nullptr;
};
GraphCache& graph_cache() {
  static GraphCache c;
  return c;
}

template <class StepFn>
int32_t md_interval_graph(const tess_model_desc* d, const float* weights, int32_t n,
                          const float box[3], float* pos, float* vel, int32_t* species,
                          const float* mass, float dt, float half_skin2, float* forces,
                          int32_t* row_ptr, uint32_t* col_shift, int32_t* rev, int64_t edge_cap,
                          void* ws, const tess_md_options& opt, bool has_epot, int32_t k,
                          hipStream_t st, StepFn step, bool* done) {
  GraphKey key;
  std::memset(&key, 0, sizeof(key));
  // the model description and the box are host arrays: their values are part of the key
  const void* ps[10] = {weights, pos, vel, species, mass, forces, row_ptr, col_shift, rev, ws};
  for (int a = 0; a < 10; a++) key.p[a] = ps[a];
  key.i[0] = n; key.i[1] = edge_cap; key.i[2] = k;
  key.i[3] = d->n_species; key.i[4] = d->n_layers;
  key.i[5] = ((int64_t)d->channels << 40) | ((int64_t)d->radial_hidden << 24) |
             ((int64_t)d->n_rbf << 16) | ((int64_t)d->l_max << 8) | d->n_heads;
  key.i[6] = opt.thermostat;
  key.i[7] = has_epot;
  key.i[8] = opt.ke_trace != nullptr;
  key.i[9] = opt.rmin_trace != nullptr;
  key.f[0] = dt; key.f[1] = box[0]; key.f[2] = box[1]; key.f[3] = box[2]; key.f[4] = d->r_cut;
  key.f[5] = opt.t_target_K; key.f[6] = opt.tau_fs; key.f[7] = half_skin2;
  GraphCache& c = graph_cache();
  std::lock_guard<std::mutex> g(c.mu);
  if (!(c.valid && c.key == key)) {
    if (c.valid) {
      (void)hipGraphExecDestroy(c.exec);
      c.valid = false;
    }
    if (hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal) != hipSuccess) {
      (void)hipGetLastError();
      return TESS_OK;  // not capturable: the caller runs the steps eagerly
    }
    int32_t rc = TESS_OK;
    for (int32_t j = 0; j < k && rc == TESS_OK; j++) rc = step(j);
    hipGraph_t graph = nullptr;
    const hipError_t ec = hipStreamEndCapture(st, &graph);
    if (rc != TESS_OK || ec != hipSuccess || !graph) {
      if (graph) (void)hipGraphDestroy(graph);
      (void)hipGetLastError();
      return rc != TESS_OK ? rc : TESS_ERR_HIP;
    }
    const hipError_t ei = hipGraphInstantiate(&c.exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess) return TESS_ERR_HIP;
    c.key = key;
    c.valid = true;
  }
  TESS_HIP_CHECK(hipGraphLaunch(c.exec, st));
  *done = true;
  return TESS_OK;
}

// Reads the status word and the skin flag (one synchronisation); returns the status error,
// else TESS_ERR_SKIN if the flag is set, else TESS_OK. A reported status is cleared.
int32_t md_sync_check(const Layout& L, hipStream_t st) {
  int32_t sf[2] = {0, 0};  // status word, skin flag
  TESS_HIP_CHECK(hipMemcpyAsync(sf, L.status, sizeof(sf), hipMemcpyDeviceToHost, st));
  TESS_HIP_CHECK(hipStreamSynchronize(st));
  const int32_t bits = sf[0], f = sf[1];
  if (bits) {
    TESS_HIP_CHECK(hipMemsetAsync(L.status, 0, sizeof(int32_t), st));
    return status_error(bits);
  }
  return f ? TESS_ERR_SKIN : TESS_OK;
}
}  // namespace

extern "C" {

int32_t tess_abi_version(void) { return 2; }

int32_t tess_timing_enable(int32_t on) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  for (auto& kv : t.ev)
    for (auto& pr : kv.second) {
      (void)hipEventDestroy(pr.first);
      (void)hipEventDestroy(pr.second);
    }
  t.ev.clear();
  for (auto& kv : t.open) (void)hipEventDestroy(kv.second);
  t.open.clear();
  t.on = on != 0;
  return TESS_OK;
}

int32_t tess_set_curve(int32_t curve) {
  if (curve != 0 && curve != 1) return TESS_ERR_ARG;
  g_curve.store(curve);
  return TESS_OK;
}

int32_t tess_timing_only(const char* kernel) {
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  t.only = kernel ? kernel : "";
  return TESS_OK;
}

int32_t tess_timing_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return TESS_ERR_ARG;
  TimingState& t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  *total_ms = 0.0;
  *launches = 0;
  auto it = t.ev.find(kernel);
  if (it == t.ev.end()) return TESS_OK;
  for (auto& pr : it->second) {
    if (hipEventSynchronize(pr.second) != hipSuccess) return TESS_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess) return TESS_ERR_HIP;
    *total_ms += ms;
    *launches += 1;
  }
  return TESS_OK;
}

const char* tess_status_string(int32_t s) {
  switch (s) {
    case TESS_OK: return "ok";
    case TESS_ERR_ARG: return "invalid argument or unsupported model shape";
    case TESS_ERR_BOX: return "box edge must exceed 2 (r_cut + skin)";
    case TESS_ERR_CAPACITY: return "neighbour list longer than edge_cap";
    case TESS_ERR_WORKSPACE: return "workspace smaller than tess_workspace_bytes()";
    case TESS_ERR_HIP: return "HIP runtime error";
    case TESS_ERR_SKIN: return "an atom moved more than skin/2 since the last rebuild";
    case TESS_ERR_SPECIES: return "species index out of range";
    case TESS_ERR_NONFINITE: return "non-finite position, energy or force";
    case TESS_ERR_ROW: return "an atom has more than 1024 candidate neighbours";
    case TESS_ERR_RADIAL: return "radial network too rough for the interpolation table";
    default: return "unknown status";
  }
}

int64_t tess_weights_count(const tess_model_desc* d) {
  if (!d || !ef_shape_supported(*d)) return -1;
  int64_t C = d->channels, R = d->radial_hidden, K = d->n_rbf, Lm = d->l_max;
  int64_t P = Lm == 1 ? 4 : 11;
  int64_t per = 2 * C * C + R * K + P * R + C * (1 + Lm) * C + Lm * C * C;
  return (int64_t)d->n_species * C + d->n_layers * per + C;
}

int64_t tess_workspace_bytes(const tess_model_desc* d, int32_t n, int64_t edge_cap) {
  if (n < 0 || edge_cap < 0) return -1;
  if (d && !ef_shape_supported(*d)) return -1;
  return layout(nullptr, d, n, edge_cap).total;
}

int32_t tess_build_neighbors(int32_t n, const float box[3], float r_cut, float skin, float* pos,
                             int32_t* species, float* vel, float* ref_pos, int32_t* perm,
                             uint32_t* hkey, int32_t* row_ptr, uint32_t* col_shift, int32_t* rev,
                             int64_t edge_cap, int64_t* n_edges, void* workspace,
                             int64_t ws_bytes, void* hip_stream) {
  if (n < 0 || n >= (1 << 27) || !box || !n_edges || edge_cap < 0 || !(r_cut > 0.0f) ||
      !(skin >= 0.0f))
    return TESS_ERR_ARG;
  if (n > 0 && (!pos || !species || !perm || !row_ptr || (!col_shift && edge_cap > 0)))
    return TESS_ERR_ARG;
  if (!box_ok(box, r_cut, skin)) return TESS_ERR_BOX;
  Layout L = layout(reinterpret_cast<char*>(workspace), nullptr, n, edge_cap);
  if (!workspace || !aligned16(workspace) || ws_bytes < L.total) return TESS_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  *n_edges = 0;
  if (n == 0) {
    if (row_ptr) TESS_HIP_CHECK(hipMemsetAsync(row_ptr, 0, sizeof(int32_t), st));
    return TESS_OK;
  }
  return build_neighbors_impl(n, box, r_cut, skin, pos, species, vel, ref_pos, nullptr, nullptr,
                              perm, hkey, row_ptr, col_shift, rev, edge_cap, n_edges, L.nbr,
                              L.status, st);
}

int32_t tess_build_neighbors_static(int32_t n, const float box[3], float r_cut, float skin,
                                    float* pos, int32_t* species, float* vel, float* ref_pos,
                                    int32_t* perm, uint32_t* hkey, int32_t* row_ptr,
                                    uint32_t* col_shift, int32_t* rev, int64_t edge_cap,
                                    int64_t* n_edges, void* hip_stream) {
  if (n < 0 || n >= (1 << 27) || !box || !n_edges || edge_cap < 0 || !(r_cut > 0.0f) ||
      !(skin >= 0.0f))
    return TESS_ERR_ARG;
  if (n > 0 && (!pos || !species || !perm || !row_ptr || (!col_shift && edge_cap > 0)))
    return TESS_ERR_ARG;
  if (!box_ok(box, r_cut, skin)) return TESS_ERR_BOX;
  // the scratch this call needs: the status word and the rebuild arrays for n atoms
  Carver need{nullptr, 0};
  (void)need.take<int32_t>(64);
  (void)carve_nbr(need, n);
  if (n > kStaticMaxAtoms || need.off > kStaticScratchBytes) return TESS_ERR_WORKSPACE;
  char* base = static_scratch();
  if (!base) return TESS_ERR_HIP;
  Carver cv{base, 0};
  int32_t* status = cv.take<int32_t>(64);
  NbrWS ws = carve_nbr(cv, n);
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  *n_edges = 0;
  if (n == 0) {
    if (row_ptr) TESS_HIP_CHECK(hipMemsetAsync(row_ptr, 0, sizeof(int32_t), st));
    return TESS_OK;
  }
  // the array keeps the previous call's contents: the status word starts each call at zero
  // (every other array the rebuild reads is written or cleared by the rebuild itself)
  k_zero_i32<<<1, 1, 0, st>>>(status);
  TESS_HIP_CHECK(hipGetLastError());
  return build_neighbors_impl(n, box, r_cut, skin, pos, species, vel, ref_pos, nullptr, nullptr,
                              perm, hkey, row_ptr, col_shift, rev, edge_cap, n_edges, ws, status,
                              st);
}

int32_t tess_check_status(void* workspace, int64_t ws_bytes, void* hip_stream) {
  if (!workspace || !aligned16(workspace) || ws_bytes < (int64_t)sizeof(int32_t))
    return TESS_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  int32_t* status = reinterpret_cast<int32_t*>(workspace);  // first word of every layout
  int32_t bits = 0;
  TESS_HIP_CHECK(hipMemcpyAsync(&bits, status, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  TESS_HIP_CHECK(hipStreamSynchronize(st));
  if (bits) TESS_HIP_CHECK(hipMemsetAsync(status, 0, sizeof(int32_t), st));
  return status_error(bits);
}

int32_t tess_energy_forces(const tess_model_desc* d, const float* weights, int32_t n,
                           const float box[3], const float* pos, const int32_t* species,
                           const int32_t* row_ptr, const uint32_t* col_shift, const int32_t* rev,
                           int64_t n_edges, double* energy, float* e_atom, float* forces,
                           void* workspace, int64_t ws_bytes, void* hip_stream) {
  if (!d || !ef_shape_supported(*d)) return TESS_ERR_ARG;
  if (n < 0 || n >= (1 << 27) || n_edges < 0 || !box || !energy || !weights || !aligned16(weights))
    return TESS_ERR_ARG;
  if (n > 0 && (!pos || !species || !row_ptr || (n_edges > 0 && !col_shift))) return TESS_ERR_ARG;
  for (int a = 0; a < 3; a++)
    if (!(box[a] > 0.0f)) return TESS_ERR_BOX;
  Layout L = layout(reinterpret_cast<char*>(workspace), d, n, n_edges);
  if (!workspace || !aligned16(workspace) || ws_bytes < L.total) return TESS_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  if (n == 0) {  // a kernel rather than a memset node, so the call stays capturable
    k_zero_f64<<<1, 1, 0, st>>>(energy);
    TESS_HIP_CHECK(hipGetLastError());
    return TESS_OK;
  }
  return ef_dispatch(*d, weights, n, box, pos, species, row_ptr, col_shift, rev, n_edges, n_edges,
                     energy, e_atom, forces, L.ef, L.ef_bytes, L.status, st);
}

int32_t tess_md_steps_ex(const tess_model_desc* d, const float* weights, int32_t n,
                         const float box[3], float r_cut, float skin, float* pos, float* vel,
                         int32_t* species, const float* mass_by_species, float dt_fs,
                         int32_t n_steps, int32_t rebuild_every, int32_t flags,
                         int32_t* perm_accum, float* forces, double* epot_trace,
                         int32_t* row_ptr, uint32_t* col_shift, int32_t* rev, int64_t edge_cap,
                         int64_t* n_edges, void* workspace, int64_t ws_bytes,
                         const tess_md_options* opt_in, void* hip_stream) {
  if (!d || !ef_shape_supported(*d)) return TESS_ERR_ARG;
  if (n < 1 || n >= (1 << 27) || n_steps < 0 || rebuild_every < 1 || edge_cap < 0 || !box ||
      !n_edges || !weights || !aligned16(weights) || !pos || !vel || !species ||
      !mass_by_species || !perm_accum ||
      !forces || !row_ptr || !col_shift || !rev || !(dt_fs > 0.0f) || !(r_cut > 0.0f) ||
      !(skin >= 0.0f) || d->r_cut != r_cut || (flags & ~(TESS_MD_FORCES_VALID | TESS_MD_GRAPH)))
    return TESS_ERR_ARG;
  tess_md_options opt{TESS_THERMOSTAT_NONE, 0.0f, 0.0f, nullptr, nullptr};
  if (opt_in) opt = *opt_in;
  if (opt.thermostat != TESS_THERMOSTAT_NONE &&
      (opt.thermostat != TESS_THERMOSTAT_BERENDSEN || !(opt.tau_fs >= dt_fs) ||
       !(opt.t_target_K >= 0.0f) || !std::isfinite(opt.t_target_K) ||
       !std::isfinite(opt.tau_fs)))
    return TESS_ERR_ARG;
  if (!box_ok(box, r_cut, skin)) return TESS_ERR_BOX;
  Layout L = layout(reinterpret_cast<char*>(workspace), d, n, edge_cap);
  if (!workspace || !aligned16(workspace) || ws_bytes < L.total) return TESS_ERR_WORKSPACE;
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  const float half_skin2 = 0.25f * skin * skin;
  const bool forces_valid = (flags & TESS_MD_FORCES_VALID) != 0;
  // graph replay needs a capturable stream and no per-launch timing events
  const bool use_graph = (flags & TESS_MD_GRAPH) != 0 && st != nullptr && !timing_on();
  const bool berendsen = opt.thermostat == TESS_THERMOSTAT_BERENDSEN;
  const bool need_ke = berendsen || opt.ke_trace;
  const bool end_kernel = need_ke || opt.rmin_trace;
  const int32_t nb = gridn(n, 256);
  int64_t ne = *n_edges;
  TESS_HIP_CHECK(hipMemsetAsync(L.flag, 0, sizeof(int32_t), st));
  if (opt.rmin_trace) {
    k_set_u32<<<1, 1, 0, st>>>(L.rmin2_bits, 0x7f800000u);
    TESS_HIP_CHECK(hipGetLastError());
  }
  // one velocity-Verlet step; `grid_edges` sizes the edge-kernel grids (the kernels stop at
  // the device-side active-edge count, so any value >= the pair count gives the same result);
  // ep/ke/rm receive the step's traces (ke/rm nullable)
  const int32_t S = d->n_species;
  auto step = [&](int64_t grid_edges, double* ep, double* ke, float* rm) -> int32_t {
    k_vv_kick_drift<<<nb, 256, 0, st>>>(n, dt_fs, forces, species, mass_by_species, S, pos, vel,
                                        L.ref_pos, half_skin2, L.flag);
    TESS_HIP_CHECK(hipGetLastError());
    int32_t rc = ef_dispatch(*d, weights, n, box, pos, species, row_ptr, col_shift, rev,
                             grid_edges, edge_cap, ep, nullptr, forces, L.ef, L.ef_bytes,
                             L.status, st, opt.rmin_trace ? L.rmin2_bits : nullptr);
    if (rc != TESS_OK) return rc;
    if (need_ke)
      k_vv_kick_ke<<<nb, 256, 0, st>>>(n, dt_fs, forces, species, mass_by_species, S, vel,
                                       L.ke_part);
    else
      k_vv_kick<<<nb, 256, 0, st>>>(n, dt_fs, forces, species, mass_by_species, S, vel);
    TESS_HIP_CHECK(hipGetLastError());
    if (end_kernel) {
      k_md_thermo<<<berendsen ? nb : 1, 256, 0, st>>>(
          n, need_ke ? nb : 0, L.ke_part, berendsen ? 1 : 0,
          berendsen ? (double)dt_fs / (double)opt.tau_fs : 0.0, (double)opt.t_target_K, vel,
          ke, L.rmin2_bits, rm);
      TESS_HIP_CHECK(hipGetLastError());
    }
    return TESS_OK;
  };
  for (int32_t s = 0; s < n_steps;) {
    if (s > 0) {
      const int32_t rc0 = md_sync_check(L, st);
      if (rc0 != TESS_OK) return rc0;
    }
    int32_t rc = build_neighbors_impl(n, box, r_cut, skin, pos, species, vel, L.ref_pos,
                                      (forces_valid || s > 0) ? forces : nullptr, perm_accum,
                                      L.perm, nullptr, row_ptr, col_shift, rev, edge_cap, &ne,
                                      L.nbr, L.status, st);
    *n_edges = ne;
    if (rc != TESS_OK) return rc;
    if (s == 0 && !forces_valid) {
      rc = ef_dispatch(*d, weights, n, box, pos, species, row_ptr, col_shift, rev, ne, edge_cap,
                       L.epot, nullptr, forces, L.ef, L.ef_bytes, L.status, st);
      if (rc != TESS_OK) return rc;
    }
    const int32_t k = n_steps - s < rebuild_every ? n_steps - s : rebuild_every;
    bool done = false;
    if (use_graph && k <= kTraceStage) {
      // the graph writes the traces into the workspace's staging arrays (fixed addresses)
      rc = md_interval_graph(
          d, weights, n, box, pos, vel, species, mass_by_species, dt_fs, half_skin2, forces,
          row_ptr, col_shift, rev, edge_cap, workspace, opt, epot_trace != nullptr, k, st,
          [&](int32_t j) {
            return step(edge_cap, L.epot_stage + j, opt.ke_trace ? L.ke_stage + j : nullptr,
                        opt.rmin_trace ? L.rmin_stage + j : nullptr);
          },
          &done);
      if (rc != TESS_OK) return rc;
      if (done && (epot_trace || opt.ke_trace || opt.rmin_trace)) {
        k_copy_traces<<<gridn(k, 256), 256, 0, st>>>(
            k, L.epot_stage, epot_trace ? epot_trace + s : nullptr, L.ke_stage,
            opt.ke_trace ? opt.ke_trace + s : nullptr, L.rmin_stage,
            opt.rmin_trace ? opt.rmin_trace + s : nullptr);
        TESS_HIP_CHECK(hipGetLastError());
      }
    }
    if (!done)
      for (int32_t j = 0; j < k; j++) {
        rc = step(ne, epot_trace ? epot_trace + s + j : L.epot,
                  opt.ke_trace ? opt.ke_trace + s + j : nullptr,
                  opt.rmin_trace ? opt.rmin_trace + s + j : nullptr);
        if (rc != TESS_OK) return rc;
      }
    s += k;
  }
  return md_sync_check(L, st);
}

int32_t tess_md_steps(const tess_model_desc* d, const float* weights, int32_t n, const float box[3],
                      float r_cut, float skin, float* pos, float* vel, int32_t* species,
                      const float* mass_by_species, float dt_fs, int32_t n_steps,
                      int32_t rebuild_every, int32_t flags, int32_t* perm_accum, float* forces,
                      double* epot_trace, int32_t* row_ptr, uint32_t* col_shift, int32_t* rev,
                      int64_t edge_cap, int64_t* n_edges, void* workspace, int64_t ws_bytes,
                      void* hip_stream) {
  return tess_md_steps_ex(d, weights, n, box, r_cut, skin, pos, vel, species, mass_by_species,
                          dt_fs, n_steps, rebuild_every, flags, perm_accum, forces, epot_trace,
                          row_ptr, col_shift, rev, edge_cap, n_edges, workspace, ws_bytes,
                          nullptr, hip_stream);
}

}  // extern "C"
