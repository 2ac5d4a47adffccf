/* tess_oracle.h -- fp64 CPU oracle for the Tessera hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
 * baseline leg may load this library. It shares no code, header, table or constant with
 * the GPU library; both read the same seeded inputs.
 *
 * The method is the one named by "Ab Initio Accuracy Beyond the Cutoff: Distributed
 * Message-Passing Equivariant Attention at Tens-of-Millions-of-Atom Scale" (Tessera,
 * abstract): atoms ordered along a space-filling curve, a neighbour list with a
 * conservative skin, and an equivariant message-passing attention potential whose forces
 * come from back-propagation. The pages name these parts without defining them; every
 * concrete definition below is the reading recorded with the function.
 */
#ifndef TESS_ORACLE_H
#define TESS_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { TOR_OK = 0, TOR_ERR_ARG = -1, TOR_ERR_BOX = -2, TOR_ERR_CAPACITY = -3,
       TOR_ERR_SKIN = -6, TOR_ERR_SPECIES = -7 };

typedef struct {
  int32_t n_species, n_layers, channels, l_max, n_heads, n_rbf, radial_hidden;
  float r_cut;
} tor_model;

int32_t tor_abi_version(void);
/* Threads used by the oracle's parallel loops. */
int32_t tor_num_threads(void);

/* Wrap one fp32 coordinate into [0, L] in fp64 and round back to fp32. */
float tor_wrap1(float x, double L);
/* Hilbert index of integer cell coordinates (each < 2^bits), 3*bits-bit key. */
uint32_t tor_hilbert_key3(uint32_t x, uint32_t y, uint32_t z, int32_t bits);
/* Wrap every coordinate and compute its 30-bit key (10 bits per axis). */
void tor_wrap_keys(int32_t n, const float box[3], const float* pos_in, float* pos_out,
                   uint32_t* keys);
/* Stable ascending argsort of 32-bit keys (ties keep ascending index). */
void tor_stable_argsort_u32(int32_t n, const uint32_t* keys, int32_t* perm);

/* Candidate list of (already wrapped, sorted) fp32 positions at r_cut+skin.
 * method 0: all-pairs scan, 1: cell list. Rows hold j ascending; entries are
 * j | code<<27 with code = 9(sx+1)+3(sy+1)+(sz+1). Returns TOR_ERR_CAPACITY with
 * *n_edges = required count when cap is too small (col_shift may be NULL then). */
int32_t tor_neighbors(int32_t n, const float box[3], const float* pos, float r_cut,
                      float skin, int32_t method, int64_t cap, int32_t* row_ptr,
                      uint32_t* col_shift, int64_t* n_edges);
/* Pairs (i<j) whose minimum-image distance lies within `band` of r_cut+skin. */
int64_t tor_flagged_pairs(int32_t n, const float box[3], const float* pos, float r_cut,
                          float skin, double band, int64_t cap, int32_t* fi, int32_t* fj);

/* Whole rebuild: wrap, keys, stable sort, permute (pos, species, optional vel/ref), CSR.
 * perm[k] = pre-call index of the atom now at slot k. */
int32_t tor_build_neighbors(int32_t n, const float box[3], float r_cut, float skin,
                            float* pos, int32_t* species, double* vel, int32_t* perm,
                            uint32_t* keys_sorted, int64_t cap, int32_t* row_ptr,
                            uint32_t* col_shift, int64_t* n_edges);

int32_t tor_n_paths(int32_t l_max);
/* Real spherical harmonics (component normalised), D=(l_max+1)^2 values. */
void tor_sph(int32_t l_max, const double n[3], double* Y);
/* Path list (l1,l2,l3 triples) and normalised coupling tensors C^p[m1][m2][m3]
 * stored densely as [P][5][5][5]. */
void tor_paths(int32_t l_max, int32_t* l1, int32_t* l2, int32_t* l3);
void tor_coupling(int32_t l_max, double* cg);

int64_t tor_weights_count(const tor_model* m);

/* Energy and forces (fp64). pos double[n][3] in the CSR's order; forces = -dE/dx.
 * e_atom (nullable) receives per-atom energies; feats (nullable) receives the final
 * node features [n][C][D]. */
int32_t tor_energy_forces(const tor_model* m, const float* weights, int32_t n,
                          const float box[3], const double* pos, const int32_t* species,
                          const int32_t* row_ptr, const uint32_t* col_shift,
                          double* energy, double* e_atom, double* forces, double* feats);

/* Velocity-Verlet between rebuilds (see tor_md_steps in the source for the exact loop);
 * thermostat 0 = NVE, 1 = Berendsen coupling to t_target_K with time constant tau_fs;
 * ke_trace / rmin_trace (nullable) receive the kinetic energy (eV) and the shortest pair
 * distance below r_cut (A) of every step. */
int32_t tor_md_steps(const tor_model* m, const float* weights, int32_t n, const float box[3],
                     float r_cut, float skin, double* pos, double* vel, int32_t* species,
                     const double* mass_by_species, double dt_fs, int32_t n_steps,
                     int32_t rebuild_every, int32_t* perm_accum, double* forces,
                     int32_t forces_valid, double* epot_trace, int64_t cap, int32_t thermostat,
                     double t_target_K, double tau_fs, double* ke_trace, double* rmin_trace);

#ifdef __cplusplus
}
#endif
#endif
