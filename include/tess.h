/* tess.h -- C ABI of libtess.so, the MI355X (gfx950) hot path of the Tessera potential.
 *
 * Method: "Ab Initio Accuracy Beyond the Cutoff: Distributed Message-Passing Equivariant
 * Attention at Tens-of-Millions-of-Atom Scale" (Tessera), abstract: atoms are ordered along
 * a space-filling curve, a three-level neighbour search with a conservative skin fixes the
 * pair topology between rebuilds, an equivariant message-passing attention potential gives
 * the energy, and forces come from back-propagation through the layers.
 *
 * Conventions shared by every entry point
 *  - Units: A, eV, fs, amu. Boxes are orthorhombic and periodic; box[3] is a HOST array.
 *  - All other array arguments are DEVICE pointers (e.g. torch tensors on cuda:0), owned by
 *    the caller, row-major, without padding. The library never allocates device memory: the
 *    caller passes a workspace of at least tess_workspace_bytes() bytes.
 *  - The weights blob and the workspace must be 16-byte aligned (torch allocations are);
 *    otherwise TESS_ERR_ARG (weights) or TESS_ERR_WORKSPACE (workspace).
 *  - `hip_stream` is a hipStream_t (NULL = default stream). Work is enqueued on it in order.
 *    tess_energy_forces and tess_md_steps also run independent kernels of the pass on one
 *    second stream per host thread and device, created by the library on its first call
 *    outside stream capture and kept until the process ends (default priority, non-blocking);
 *    it forks from and joins `hip_stream` through events, so the pass stays ordered on
 *    `hip_stream` (and captures into one graph). A call that is the thread's first on a
 *    device and runs under capture uses `hip_stream` alone.
 *  - Return value: a tess_status. Argument, box and workspace errors are detected on the host
 *    before anything is enqueued. TESS_ERR_HIP reports a failed HIP call (the stream state is
 *    then undefined).
 *  - Device status word: the first 4 bytes of the workspace. Kernels record problems they
 *    find on the device there (asynchronously): a species index outside [0, n_species) seen
 *    by the energy pass, and a non-finite position (neighbour build), energy or force (energy
 *    pass), and a radial network whose interpolation table deviates from it by more than
 *    1e-6 of max|w| or 1e-4 of max|dw/dr| at the knot intervals' midpoints (energy pass; the
 *    radial weights are interpolated from a per-call table of 1,024 intervals on [0, r_cut]).
 *    The next synchronising call on that workspace -- tess_check_status,
 *    tess_build_neighbors or tess_md_steps -- returns TESS_ERR_SPECIES (first),
 *    TESS_ERR_NONFINITE or TESS_ERR_RADIAL and clears the word. A fresh workspace must start with that word zero
 *    (zero-filled memory, or one tess_check_status call); the rest of the workspace may hold
 *    anything, since the library writes every other value there before reading it. The Tessera abstract reports runs
 *    with no broken bonds or anomalously close pairs; this is the device-side check that a
 *    run has not blown up.
 *  - Supported model shapes (kernels are compiled per shape): n_rbf == 8, n_species <= 16,
 *    n_layers <= 16 and (l_max, channels, n_heads, radial_hidden) one of (1, 16, 1, 32),
 *    (1, 32, 4, 32), (2, 16, 4, 32), (2, 32, 4, 32), (2, 64, 4, 64). Others: TESS_ERR_ARG.
 *  - Limits: n_atoms < 2^27; at most 1024 candidate neighbours per atom.
 */
#ifndef TESS_H
#define TESS_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TESS_OK = 0,
  TESS_ERR_ARG = -1,       /* bad argument or unsupported model shape */
  TESS_ERR_BOX = -2,       /* some box edge <= 2 (r_cut + skin) */
  TESS_ERR_CAPACITY = -3,  /* candidate list longer than edge_cap (see *n_edges) */
  TESS_ERR_WORKSPACE = -4, /* workspace smaller than tess_workspace_bytes() */
  TESS_ERR_HIP = -5,       /* a HIP runtime call failed */
  TESS_ERR_SKIN = -6,      /* an atom moved more than skin/2 since the last rebuild */
  TESS_ERR_SPECIES = -7,   /* species index outside [0, n_species) (device status word) */
  TESS_ERR_NONFINITE = -8, /* non-finite position, energy or force (device status word) */
  TESS_ERR_ROW = -9,       /* an atom has more than 1024 candidate neighbours */
  TESS_ERR_RADIAL = -10    /* radial network too rough for the interpolation table (status word) */
} tess_status;

/* Model hyper-parameters. Paths P follow from l_max (4 for l_max 1, 11 for l_max 2). */
typedef struct {
  int32_t n_species, n_layers, channels, l_max, n_heads, n_rbf, radial_hidden;
  float r_cut;
} tess_model_desc;

int32_t tess_abi_version(void); /* 2 */
const char* tess_status_string(int32_t status);

/* tess_check_status -- synchronises `hip_stream`, reads and clears the device status word of
 * `workspace` (any workspace of tess_workspace_bytes(); at least 4 bytes, 16-byte aligned).
 * Returns TESS_OK, TESS_ERR_SPECIES, TESS_ERR_NONFINITE or TESS_ERR_RADIAL
 * (TESS_ERR_WORKSPACE for a bad pointer or size). */
int32_t tess_check_status(void* workspace, int64_t ws_bytes, void* hip_stream);

/* Number of fp32 weights. Blob order (row-major [out][in], y = W x): Emb[S][C]; for each
 * layer W_q[C][C], W_k[C][C], W1[R][K], W2[P][R], W_lin0[C(1+l_max)][C], then W_lin^l[C][C]
 * for l = 1..l_max; finally w_E[C]. Returns -1 for an unsupported shape. */
int64_t tess_weights_count(const tess_model_desc* desc);

/* Workspace bytes for any entry point at this size (desc may be NULL for the neighbour
 * build alone). */
int64_t tess_workspace_bytes(const tess_model_desc* desc, int32_t n_atoms, int64_t edge_cap);

/* tess_build_neighbors -- the three-level neighbour search of the Tessera abstract:
 * (1) wrap every coordinate into the box (fp64, then rounded to fp32) and order the atoms by
 *     a 30-bit Hilbert key (10 bits per axis, Skilling's transpose form) with a stable
 *     radix sort; (2) bin the sorted atoms into cells no narrower than r_cut+skin;
 * (3) keep the pairs with |x_j - x_i + s L|^2 < (r_cut+skin)^2 (fp64, minimum image s),
 *     rows listing j in ascending order.
 *  in/out  pos[n][3]     positions; on return wrapped into [0, L] and in sorted order
 *  in/out  species[n]    permuted to sorted order
 *  in/out  vel[n][3]     nullable; permuted to sorted order
 *  out     ref_pos[n][3] nullable; receives a copy of the returned positions
 *  out     perm[n]       perm[k] = pre-call index of the atom now at slot k
 *  out     hkey[n]       nullable; Hilbert key of each sorted atom
 *  out     row_ptr[n+1], col_shift[edge_cap]: CSR; entry = j | code<<27 with
 *          code = 9(sx+1) + 3(sy+1) + (sz+1) the image shift s in {-1,0,1}^3
 *  out     rev[edge_cap] nullable; rev[e] = slot of the reverse pair (j <- i, -s)
 *  out     *n_edges (HOST) number of pairs; on TESS_ERR_CAPACITY the required count
 *          (a count above 2^31 - 1, which the int32 row offsets cannot hold, is also reported
 *          as TESS_ERR_CAPACITY with the true count: no edge_cap satisfies it)
 * Synchronises the stream once (to read the pair count and the device status word). On
 * TESS_ERR_CAPACITY / TESS_ERR_ROW the positions and permutation outputs are valid but
 * col_shift and rev are not. A set status word (a non-finite input coordinate, or a problem
 * left by an earlier energy pass on this workspace) is returned as TESS_ERR_NONFINITE /
 * TESS_ERR_SPECIES and cleared; col_shift and rev are then not written. */
int32_t tess_build_neighbors(int32_t n, const float box[3], float r_cut, float skin,
                             float* pos, int32_t* species, float* vel, float* ref_pos,
                             int32_t* perm, uint32_t* hkey, int32_t* row_ptr,
                             uint32_t* col_shift, int32_t* rev, int64_t edge_cap,
                             int64_t* n_edges, void* workspace, int64_t ws_bytes,
                             void* hip_stream);

/* tess_build_neighbors_static -- tess_build_neighbors for callers that cannot allocate
 * memory (no hipMalloc and no workspace of their own: code run under stream capture, tight
 * serving loops, harnesses that forbid allocation). The arguments, outputs, synchronisation
 * and errors are those of tess_build_neighbors, without the workspace: the rebuild's scratch
 * is a 48 MiB array inside the library, one per GPU, kept until the process ends (the call
 * itself allocates nothing). Limit: n <= 524288 atoms, else TESS_ERR_WORKSPACE before anything
 * is enqueued. Every call on one GPU shares that GPU's array, so calls that overlap on one GPU
 * (concurrent streams or threads) race; serialise them. Its status word starts every call at
 * zero, so only this call's own non-finite coordinates are reported. */
int32_t tess_build_neighbors_static(int32_t n, const float box[3], float r_cut, float skin,
                                    float* pos, int32_t* species, float* vel, float* ref_pos,
                                    int32_t* perm, uint32_t* hkey, int32_t* row_ptr,
                                    uint32_t* col_shift, int32_t* rev, int64_t edge_cap,
                                    int64_t* n_edges, void* hip_stream);

/* tess_energy_forces -- energy and forces of the equivariant message-passing attention
 * stack (Tessera title and abstract: equivariant attention, force back-propagation).
 * Per layer: q/k projections of the scalar channels, per-edge Bessel radial basis with a
 * cosine envelope and real spherical harmonics (l <= l_max), a radial MLP giving one weight
 * per coupling path, the coupled value A_e h_j (Gaunt-normalised Clebsch-Gordan paths), a
 * per-destination softmax over edges inside r_cut weighted by the envelope, sum
 * aggregation, and a gated residual update. E = sum_i w_E . h_i^(T, l=0); F = -dE/dx.
 *  in  weights  fp32 blob (tess_weights_count), pos[n][3] in the CSR's atom order,
 *      species[n], row_ptr/col_shift/rev from tess_build_neighbors (rev may be NULL: it is
 *      then rebuilt in the workspace), n_edges = row_ptr[n].
 *  out energy   device double[1]; e_atom device float[n] (nullable);
 *      forces   device float[n][3] (nullable: energy only, no backward pass).
 * Fully asynchronous (no host synchronisation). Species outside [0, n_species) are clamped
 * into that range where they index the weights (no access leaves the weights) and set
 * TESS_ERR_SPECIES in the workspace's device status word; a non-finite energy or force sets
 * TESS_ERR_NONFINITE there. Both are reported by the next synchronising call
 * (tess_check_status, tess_build_neighbors, tess_md_steps). */
int32_t tess_energy_forces(const tess_model_desc* desc, const float* weights, int32_t n,
                           const float box[3], const float* pos, const int32_t* species,
                           const int32_t* row_ptr, const uint32_t* col_shift,
                           const int32_t* rev, int64_t n_edges, double* energy,
                           float* e_atom, float* forces, void* workspace, int64_t ws_bytes,
                           void* hip_stream);

#define TESS_MD_FORCES_VALID 1 /* forces[] already holds F(pos) in the current order */
#define TESS_MD_GRAPH 2        /* replay each interval's steps from a captured HIP graph */

/* tess_md_steps -- velocity-Verlet MD with a neighbour rebuild every `rebuild_every` steps
 * (Tessera abstract: a conservative skin keeps the topology between rebuilds). For
 * s = 0..n_steps-1: if s % rebuild_every == 0, rebuild (pos, vel, species, forces and
 * perm_accum are permuted to the new order; ref positions reset), computing the forces
 * first when s == 0 and TESS_MD_FORCES_VALID is not set; then v += dt/2 F/m, x += dt v
 * (x is not re-wrapped between rebuilds), F = -dE/dx (epot_trace[s] = E), v += dt/2 F/m,
 * with F/m converted by 9.648533e-3 (eV/A/amu -> A/fs^2).
 *  in     mass_by_species device float[n_species] (amu), dt_fs, n_steps, rebuild_every
 *  in/out pos, vel, species, perm_accum[n] (perm_accum[k] = caller id of slot k), forces[n][3]
 *  out    epot_trace device double[n_steps] (nullable); row_ptr/col_shift/rev as in
 *         tess_build_neighbors; *n_edges (HOST) pairs of the last rebuild
 * Synchronises once per rebuild. If an atom moved more than skin/2 from its position at
 * the last rebuild, the call finishes that interval and returns TESS_ERR_SKIN. At the same
 * synchronisation it reads the device status word: a species outside [0, n_species) or a
 * non-finite position, energy or force stops the run with TESS_ERR_SPECIES /
 * TESS_ERR_NONFINITE (reported before TESS_ERR_SKIN; masses are read at the species index
 * clamped into range, so no access leaves mass_by_species).
 * flags: TESS_MD_FORCES_VALID; TESS_MD_GRAPH captures the steps of a rebuild interval into a
 * HIP graph once and replays it for later intervals and calls with identical arguments
 * (pointers, sizes, step count, dt, skin, box, model, thermostat, which traces are
 * requested); results are identical to eager launches. Traces are staged in the workspace
 * and copied out after each replay, so their offsets do not force a re-capture. It is
 * ignored on the NULL stream, while kernel timing is enabled and for rebuild_every > 256.
 * One graph is cached per process (a call with other arguments re-captures it); calls that
 * use the flag must not run concurrently from several threads. Other flag bits:
 * TESS_ERR_ARG. */
int32_t tess_md_steps(const tess_model_desc* desc, const float* weights, int32_t n,
                      const float box[3], float r_cut, float skin, float* pos, float* vel,
                      int32_t* species, const float* mass_by_species, float dt_fs,
                      int32_t n_steps, int32_t rebuild_every, int32_t flags,
                      int32_t* perm_accum, float* forces, double* epot_trace,
                      int32_t* row_ptr, uint32_t* col_shift, int32_t* rev, int64_t edge_cap,
                      int64_t* n_edges, void* workspace, int64_t ws_bytes, void* hip_stream);

/* Thermostat and per-step monitors for tess_md_steps_ex (Tessera abstract: the capsid runs
 * under NVT and shows no anomalously close pairs; the pages do not name the thermostat).
 *  thermostat  TESS_THERMOSTAT_NONE: NVE, as tess_md_steps.
 *              TESS_THERMOSTAT_BERENDSEN: weak coupling (Berendsen et al., J. Chem. Phys. 81,
 *              3684, 1984) of the kinetic temperature T = 2 KE / (3 N k_B) (3N degrees of
 *              freedom, k_B = 8.617333262e-5 eV/K, KE = sum m v^2 / 2 converted to eV by
 *              1/9.648533e-3) to t_target_K: after the second half-kick of every step all
 *              velocities are multiplied by lambda = sqrt(1 + (dt/tau_fs)(t_target_K/T - 1))
 *              (lambda = 1 when T = 0). Requires tau_fs >= dt_fs and t_target_K >= 0.
 *  ke_trace    device double[n_steps] (nullable): kinetic energy in eV at the end of step s
 *              (after the thermostat), so ke_trace[s] + epot_trace[s] is the total energy.
 *  rmin_trace  device float[n_steps] (nullable): shortest distance (A) over the listed pairs
 *              with r < r_cut at the positions where step s evaluated the forces; +inf when
 *              no pair is that close.
 * KE is summed in fp64 per block of atoms and the blocks in a fixed order, so traces and
 * velocities are deterministic. */
#define TESS_THERMOSTAT_NONE 0
#define TESS_THERMOSTAT_BERENDSEN 1
typedef struct {
  int32_t thermostat;
  float t_target_K;
  float tau_fs;
  double* ke_trace;
  float* rmin_trace;
} tess_md_options;

/* tess_md_steps_ex -- tess_md_steps with a thermostat and monitors. `opt` is a HOST pointer
 * (nullable: identical to tess_md_steps); every other argument, the loop, the flags, the
 * synchronisation and the errors are those of tess_md_steps. Invalid options: TESS_ERR_ARG
 * before anything is enqueued. With TESS_MD_GRAPH the options are part of the graph's key. */
int32_t tess_md_steps_ex(const tess_model_desc* desc, const float* weights, int32_t n,
                         const float box[3], float r_cut, float skin, float* pos, float* vel,
                         int32_t* species, const float* mass_by_species, float dt_fs,
                         int32_t n_steps, int32_t rebuild_every, int32_t flags,
                         int32_t* perm_accum, float* forces, double* epot_trace,
                         int32_t* row_ptr, uint32_t* col_shift, int32_t* rev, int64_t edge_cap,
                         int64_t* n_edges, void* workspace, int64_t ws_bytes,
                         const tess_md_options* opt, void* hip_stream);

/* Space-filling curve used by later rebuilds in this process: 0 = Hilbert (default, the
 * method's), 1 = Morton (Z-order of the same 10-bit cells; for locality comparisons only, the
 * pair set is the same, the atom order and hence perm/hkey differ). Returns TESS_ERR_ARG for
 * other values. Not thread-safe with concurrent rebuilds. */
int32_t tess_set_curve(int32_t curve);

/* Optional kernel timing for benchmarks (not part of the method). tess_timing_enable(1)
 * clears the counters and, until tess_timing_enable(0), records a pair of HIP events on the
 * launching stream around each launch of the instrumented kernels ("edge_radial", "logits",
 * "edge_apply", "edge_grad", "edge_grad_last", "edge_tapply", "node_gemm", "radix_scatter",
 * "nbr_count", "nbr_fill"). tess_timing_read waits for those events and returns the summed
 * milliseconds and the launch count of one kernel. Host memory only; not thread-safe across
 * concurrent calls on several streams. */
int32_t tess_timing_enable(int32_t on);
int32_t tess_timing_read(const char* kernel, double* total_ms, int64_t* launches);
/* Restrict the timing events to one instrumented kernel (NULL or "" = all of them); an event
 * pair costs a little GPU time, so a benchmark can time only the kernel it reports. */
int32_t tess_timing_only(const char* kernel);

#ifdef __cplusplus
}
#endif
#endif
