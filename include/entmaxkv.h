/*
 * entmaxkv.h -- C ABI of the support-aware paged alpha-entmax decode library
 * for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the EntmaxKV summary page (gist.science, paper
 * 2605.21649, "EntmaxKV – Décodage Conscient du Support pour l'Attention
 * Entmax"):
 *   ekv_build_page_meta  -- per-page key metadata            (§2.A)
 *   ekv_score_pages      -- query-aware page upper bounds     (§2.A)
 *   ekv_select_pages     -- top-k or Gaussian-aware selection (§2.B)
 *   ekv_entmax_decode    -- alpha-entmax over selected pages  (§2.C)
 *   ekv_softmax_decode   -- softmax over the same pages (comparison, §3-§4)
 * The alpha-entmax mapping itself is the standard one: with
 * z_i = (alpha-1) * s_i, p_i = [z_i - tau]_+^(1/(alpha-1)) and tau chosen so
 * that sum_i p_i = 1.  tau is always reported in that z-space.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  * Every array argument is a DEVICE pointer owned by the caller; the library
 *    never allocates, frees or copies to the host, and never synchronises.
 *    Work is enqueued on `stream` (0 = the null stream) and is asynchronous.
 *  * Arguments are validated on the host before anything is launched; on any
 *    error nothing is launched and a negative ekv_status is returned.  Values
 *    that live in device memory (seq_lens, block_table, sel, n_sel) cannot be
 *    checked without a synchronisation: they must satisfy
 *        0 <= seq_lens[b] <= max_pages_per_seq * page_size,
 *        0 <= block_table[b][p] < num_phys_pages  for p < ceil(seq_lens[b]/P),
 *    and a physical page referenced by several rows must hold the same number
 *    of valid tokens in each of them.
 *  * An empty row (seq_lens[b] = 0, an idle batch slot) has no pages: the
 *    selections give it n_sel = 0 (and tau_hat NaN), the decode writes a zero
 *    output, tau NaN and n_support 0 for its heads, and the metadata calls
 *    and the append skip it.  Its block-table entries are not used.
 *  * Alignment: K, V, q, out, kmin, kmax, mean and var 16 bytes; int32 and
 *    fp32 arrays 4 bytes; fp64 arrays 8 bytes; workspaces 256 bytes.
 *  * Layouts (row-major, innermost last):
 *        K, V          [num_phys_pages][Hkv][P][d]   bf16 or fp32
 *        q, out        [B][Hq][d]                    fp32
 *        block_table   [B][max_pages_per_seq]        int32
 *        seq_lens      [B]                           int32
 *        kmin, kmax    [num_phys_pages][Hkv][d]      same dtype as K
 *        mean, var     [num_phys_pages][Hkv][d]      fp32, or bf16 with
 *                                                    compact_moments
 *    Query head h reads KV head h / (Hq/Hkv) (contiguous query groups).
 *    Token t of logical page p of row b is valid when p*P + t < seq_lens[b];
 *    invalid slots of a row's last page are never read.
 *  * Supported: head_dim in {64, 128}; page_size in {1,2,4,8,16,32,64};
 *    Hq % Hkv == 0 and Hq/Hkv in {1,2,4,8}; kv dtype bf16 or fp32.
 *  * Calls are thread-safe: the library holds no mutable global state, except
 *    the per-device scratch of ekv_decode_step_noalloc (see there).
 */
#ifndef ENTMAXKV_H
#define ENTMAXKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EKV_OK = 0,
  EKV_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad shape or value  */
  EKV_ERR_UNSUPPORTED = -2, /* valid but not implemented (dims, alpha, ...) */
  EKV_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required   */
  EKV_ERR_HIP = -4          /* a HIP launch failed (see hipGetLastError)    */
} ekv_status;

typedef enum { EKV_BF16 = 0, EKV_F32 = 1 } ekv_dtype;

typedef enum {
  EKV_SELECT_TOPK = 0,  /* fixed budget: k pages with the largest bound     */
  EKV_SELECT_GAUSS = 1,     /* Gaussian estimate tau-hat of the threshold, margin Delta;
                               a page's maximum score estimated by its box bound     */
  EKV_SELECT_GAUSS_EST = 2, /* same tau-hat and Delta; maximum score estimated as the
                               expected maximum of its tokens' Gaussian scores       */
  EKV_SELECT_GAUSS_MASS = 3 /* same tau-hat; a page is kept when its expected entmax
                               mass reaches the threshold passed as delta            */
} ekv_policy;

typedef struct {
  int32_t batch;             /* B                                           */
  int32_t num_q_heads;       /* Hq                                          */
  int32_t num_kv_heads;      /* Hkv                                         */
  int32_t head_dim;          /* d                                           */
  int32_t page_size;         /* P, tokens per page                          */
  int32_t max_pages_per_seq; /* maxP, row stride of block_table and scores  */
  int32_t num_phys_pages;    /* Np, pages in the K/V pool                   */
  int32_t kv_dtype;          /* ekv_dtype of K, V, kmin, kmax               */
  int32_t compact_moments;   /* 0: page mean/var fp32; 1: bf16 (each rounded
                                once, to nearest even, from its fp64 value) */
} ekv_cache_desc;

/*
 * Page metadata (§2.A "Notation de Page Consciente de la Requête": a
 * per-coordinate bounding box of the page's keys, and the first and second
 * moments of the keys so that in-page scores can be modelled as Gaussian).
 *
 * For each row b and logical page p with first_page[b] <= p <
 * first_page[b] + span (and p < ceil(seq_lens[b]/P)), over the page's valid
 * tokens, writes to physical page pi = block_table[b][p], KV head g:
 *   kmin[pi][g][j], kmax[pi][g][j]  exact per-coordinate min / max;
 *   mean[pi][g][j]                  (sum_t k_tj) / n in fp64, rounded to fp32;
 *   var[pi][g][j]                   population variance (1/n) sum_t (k_tj - mean)^2,
 *                                   two-pass in fp64, rounded to fp32;
 *   with desc->compact_moments = 1 both are rounded once from fp64 to the
 *   nearest bf16 instead (ties to an even last bit; half the bytes the
 *   Gaussian scorer reads for them).
 * first_page: device int32 [B] or NULL (= 0 for every row).
 * span: pages per row to (re)build; span <= 0 means max_pages_per_seq.
 *       span = 1 with first_page[b] = last page refreshes the page a decode
 *       step has just appended to.
 * mean and var may both be NULL (bounding box only).
 */
ekv_status ekv_build_page_meta(const ekv_cache_desc* desc, const void* K,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* first_page, int32_t span,
                               void* kmin, void* kmax, void* mean, void* var,
                               hipStream_t stream);

/*
 * Device-side check of the values the other entry points cannot validate on
 * the host without a synchronisation (see the conventions above): writes
 *   bad[0] = number of rows b with seq_lens[b] outside [0, max_pages_per_seq * P],
 *   bad[1] = number of entries block_table[b][p], p < ceil(seq_lens[b]/P) of a
 *            row with a valid length, outside [0, num_phys_pages).
 * bad: device int32 [2], overwritten (cleared by a kernel, so the call can be
 * captured in a graph).  Nothing is synchronised: read bad after the stream
 * has reached this call.  Meant for debugging and admission checks; the
 * decode path itself never reads it.
 */
ekv_status ekv_validate_cache(const ekv_cache_desc* desc, const int32_t* block_table,
                              const int32_t* seq_lens, int32_t* bad, hipStream_t stream);

/*
 * Decode-time append of one token per row (§2.A: the page metadata is stored
 * per page, so a new token changes only its own page's record).  For every
 * row b, with t = seq_lens[b] - 1 (seq_lens already counts the new token),
 * p = t / P, slot = t % P and pi = block_table[b][p]:
 *   K[pi][g][slot][:] = k_new[b][g][:],  V[pi][g][slot][:] = v_new[b][g][:]
 * for every KV head g, and the metadata of (pi, g) becomes that of the page's
 * slot + 1 valid tokens, exactly as ekv_build_page_meta would compute it:
 * without mean/var, the box is updated in place (a page's first token starts
 * a new box; min and max over the same tokens are the same exact values);
 * with mean/var, the page's box and moments are rebuilt from its rows.
 * Arrays: k_new, v_new [B][Hkv][d] in the K dtype (16-byte aligned); K, V,
 * kmin, kmax, mean, var as for ekv_build_page_meta.  mean and var are both
 * NULL or both set.  Rows with seq_lens[b] < 1 are skipped.  Device-side
 * preconditions (not checked): page p of every row is allocated in
 * block_table, and no other row references it (it is rewritten in place).
 * Everything else of the cache is left untouched.  One launch.
 */
ekv_status ekv_append_token(const ekv_cache_desc* desc, const void* k_new, const void* v_new,
                            const int32_t* block_table, const int32_t* seq_lens, void* K,
                            void* V, void* kmin, void* kmax, void* mean, void* var,
                            hipStream_t stream);

/*
 * Page scores (§2.A: a deterministic upper bound on the largest score any
 * token of the page can reach for the query; Gaussian moments of the scores).
 * For row b, query head h = g G + i (G = Hq/Hkv, KV head g), logical page
 * p < ceil(seq_lens[b]/P), with pi = block_table[b][p]:
 *   ub[b][g][p][i] = RN_fp32( scale * sum_j max(q_j kmin_j, q_j kmax_j) ),
 *                    accumulated in fp64 from exact products;
 *   ubg[b][g][p]   = max over i of ub[b][g][p][i];
 *   gm[b][h][p]  = scale   * sum_j q_j mean_j          (fp64),
 *   gv[b][h][p]  = scale^2 * sum_j q_j^2 var_j         (fp64).
 * Entries with p >= ceil(seq_lens[b]/P) are left untouched.
 * Arrays: q [B][Hq][d]; ub [B][Hkv][maxP][G] (page-major: the G bounds of a
 * page are adjacent); gm, gv [B][Hq][maxP]; ubg [B][Hkv][maxP].
 * ub may be NULL (only ubg written).  gm and gv are both NULL or both set;
 * when set, mean and var must be set.  scale must be finite and > 0.
 */
ekv_status ekv_score_pages(const ekv_cache_desc* desc, const float* q, float scale,
                           const void* kmin, const void* kmax,
                           const void* mean, const void* var,
                           const int32_t* block_table, const int32_t* seq_lens,
                           float* ub, float* ubg, double* gm, double* gv,
                           hipStream_t stream);

/*
 * Candidate selection (§2.B "Politiques de Sélection des Candidats").
 * Output per (row b, KV head g): sel[b][g][0 .. n_sel[b][g]) ascending logical
 * page indices; entries past n_sel are left untouched.
 *
 * EKV_SELECT_TOPK: the min(top_k, n_b) pages with the largest ubg[b][g][p];
 *   equal values go to the lower page index.  Uses ubg only.  top_k >= 1.
 * EKV_SELECT_GAUSS: per query head h, tau_hat[b][h] (fp64) is the root of
 *   sum_p n_p * E[(X_p - tau)_+^gamma] = 1,
 *   X_p ~ N((alpha-1) gm[b][h][p], (alpha-1)^2 gv[b][h][p]), n_p = valid tokens
 *   of page p, gamma = 1/(alpha-1); page p is kept when
 *   (alpha-1) * ub[b][g][p][i] >= tau_hat[b][g G + i] - delta for some i < G
 *   (compared in fp64).  If no page is kept, the page with the largest ubg is
 *   (lowest index on ties).  Needs ub, ubg, gm, gv and tau_hat; delta >= 0.
 *   alpha must lie in (1, 2] with gamma <= 64 (alpha >= 1 + 1/64), else
 *   EKV_ERR_UNSUPPORTED: for alpha > 2 (gamma < 1) the normalisation is no
 *   longer convex in tau and the monotone Newton solve does not apply.  A
 *   gamma within 1e-6 of an integer is taken as that integer; E[(X - c)_+^g]
 *   = s^g I_g((mu - c)/s), I_g(h) = E[(Z + h)_+^g], comes from the recurrence
 *   I_g = h I_{g-1} + (g-1) I_{g-2} started at I_0 = Phi, I_1 = h Phi + phi
 *   (integer g), or at I_f, I_{f+1} with f = g - floor(g), which each launch
 *   tabulates per block over h (Chebyshev pieces from a Gauss-Jacobi /
 *   Gauss-Legendre quadrature of their defining integrals, about 1e-13
 *   relative).
 * EKV_SELECT_GAUSS_EST: as EKV_SELECT_GAUSS, but the estimated maximum score
 *   of page p for head h is the expected maximum of its n_p token scores
 *   modelled as independent N(gm, gv) draws (the estimated maximum of §2.B):
 *   page p is kept when
 *   (alpha-1) * (gm[b][h][p] + e_{n_p} * sqrt(gv[b][h][p])) >= tau_hat[b][h] - delta
 *   (fp64, each operation rounded separately), with e_n = E[max of n iid
 *   N(0,1)] (e_1 = 0, e_16 = 1.76599...).  ub is not read and may be NULL.
 *   The empty-set guard and every other rule are those of EKV_SELECT_GAUSS.
 * EKV_SELECT_GAUSS_MASS: same tau_hat; instead of a maximum score, the
 *   expected entmax mass of the page's tokens under the same Gaussian model,
 *   M = n_p * E[(X_p - tau_hat[b][h])_+^gamma] (these sum to 1 over the pages
 *   at tau_hat; dropping a page drops its mass, and the output error is at
 *   most 2 B times the dropped mass, §3).  Page p is kept when M >= delta for
 *   some head of the group (fp64); delta is here the mass threshold (>= 0).
 *   ub is not read and may be NULL; guard and other rules as EKV_SELECT_GAUSS.
 * Arrays: sel [B][Hkv][maxP] int32; n_sel [B][Hkv] int32; tau_hat [B][Hq] fp64.
 */
ekv_status ekv_select_pages(const ekv_cache_desc* desc, const int32_t* seq_lens,
                            int32_t policy, int32_t top_k, float alpha, float delta,
                            const float* ub, const float* ubg,
                            const double* gm, const double* gv,
                            int32_t* sel, int32_t* n_sel, double* tau_hat,
                            hipStream_t stream);

/*
 * Sparse alpha-entmax attention over the selected pages (§2.C "Attention
 * Entmax Parcimonieuse": only the selected pages' keys and values are loaded;
 * the entmax weights are computed over that reduced set; the output is exact
 * when the set contains the full distribution's support, §3).
 * For each row b and query head h (KV head g), over the valid tokens i of the
 * pages sel[b][g][0 .. n_sel[b][g]) (all pages 0 .. n_b-1 when sel is NULL):
 * entries are logical pages of row b in [0, n_b), distinct, in any order; an
 * entry outside [0, n_b) is taken as a page with no valid token (nothing is
 * read through it).
 *   z_i   = (alpha-1) * scale * <q[b][h], k_i>           (fp32 accumulation)
 *   tau   : sum_i [z_i - tau]_+^(1/(alpha-1)) = 1         (solved in fp64)
 *   out[b][h] = sum_i p_i v_i / sum_i p_i,  p_i = [z_i - tau]_+^(1/(alpha-1))
 *   tau_out[b][h] = tau (fp32), if tau_out is not NULL;
 *   n_support[b][h] = #{i : p_i > 0} (int32), if n_support is not NULL.
 * Only value rows with p_i > 0 are read (entmax zeros are exact).
 * max_sel: host upper bound on every n_sel[b][g] (<= max_pages_per_seq; <= 0
 *   means max_pages_per_seq).  It sizes the launch and the workspace; a row
 *   whose n_sel exceeds it gets NaN outputs.
 * ub / zlb (both NULL, or both set): page pruning.  ub [B][Hkv][maxP][G] fp32
 *   holds per-head page bounds as written by ekv_score_pages or
 *   ekv_score_select_pages (ub[b][g][p][i] >= scale * <q[b][h], k> for every
 *   valid key k of page p, h = g G + i).  A first launch writes zlb[b][h]
 *   (fp32, [B][Hq]): the largest z over the valid tokens of the selected page
 *   with the largest bound for head h, lowest page on ties (a lower bound of
 *   z_max over the selected tokens; -inf if none).  The keys of a selected
 *   page are then not read when, for every head h of its group,
 *   x + 1e-3 (1 + |x|) < zlb[b][h] - 1 - 1e-4 (1 + |zlb[b][h]|) with x =
 *   (alpha-1) times its bound (fp32; the slacks exceed the rounding of the
 *   bound and of the fp32 scores): since tau >= z_max - 1 (the largest
 *   weight is at most 1), none of its tokens can carry weight, so tau, out
 *   and n_support are those of the unpruned call (§2.C, §3: only support
 *   tokens matter).  How many pages this skips depends on the data.
 * ws / ws_bytes: device scratch of at least ekv_decode_workspace_bytes(desc,
 *   max_sel) bytes, 256-byte aligned; its contents need no initialisation
 *   and are garbage afterwards.  alpha > 1 and finite; scale > 0.
 */
ekv_status ekv_entmax_decode(const ekv_cache_desc* desc, const float* q, float scale,
                             float alpha, const void* K, const void* V,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* sel, const int32_t* n_sel, int32_t max_sel,
                             const float* ub, float* zlb, float* out, float* tau_out,
                             int32_t* n_support, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/*
 * ekv_entmax_decode in one launch: the same arguments and results (up to
 * summation order), but the tau solve and the support-row gather of each
 * (row, KV head) are run by the last workgroup to finish that pair's key
 * scores (one wave per query head), instead of by a second launch.  This
 * saves a launch but holds more registers during the key stream; on the GQA
 * decode shape it measured slower than the two-launch ekv_entmax_decode,
 * which ekv_decode_step therefore uses.  Cross-workgroup data moves through
 * device-coherent loads and stores and a relaxed arrival counter.
 * ws / ws_bytes: at least ekv_decode_fused_workspace_bytes(desc, max_sel)
 *   bytes, 256-byte aligned, ZERO-FILLED before first use; every completed
 *   call leaves its arrival counters zero again, so the workspace can be
 *   reused (and the call captured in a graph) without clearing.  Calls that
 *   share a workspace must not overlap.
 */
ekv_status ekv_entmax_decode_fused(const ekv_cache_desc* desc, const float* q, float scale,
                                   float alpha, const void* K, const void* V,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* sel, const int32_t* n_sel, int32_t max_sel,
                                   const float* ub, float* zlb, float* out, float* tau_out,
                                   int32_t* n_support, void* ws, size_t ws_bytes,
                                   hipStream_t stream);

/* Scratch bytes ekv_entmax_decode_fused needs (0 if desc is invalid). */
size_t ekv_decode_fused_workspace_bytes(const ekv_cache_desc* desc, int32_t max_sel);

/*
 * Fused first half of a decode step with the top-k policy (§2.A + §2.B(1)):
 * the same results as
 *   ekv_build_page_meta(first_page = last page of each row, span = 1,
 *                       mean = var = NULL)          [only if refresh_last_page]
 *   ekv_score_pages(ub, gm = gv = NULL)  ->  ekv_select_pages(TOPK, top_k)
 * in one launch (ub may be NULL: then the per-head bounds are not written): each workgroup scores a slice of one (row, KV head)'s pages
 * (the one holding the row's last page first rebuilds that page's bounding
 * box), and the last workgroup to finish a (row, KV head) runs its top-k over
 * the bounds it finds in L2.  kmin/kmax are read (and, for the refreshed page,
 * written); mean/var are not maintained by this call.
 * ws / ws_bytes: at least ekv_score_select_workspace_bytes(desc) bytes of
 *   arrival counters, 256-byte aligned, ZERO-FILLED before first use; every
 *   completed call leaves them zero, so the workspace can be reused (and the
 *   call captured in a graph) without clearing.  Calls sharing a workspace
 *   must not overlap.
 * With refresh_last_page set, a row's last page must not be referenced by
 * another row (it is rebuilt while other rows are being scored).
 */
ekv_status ekv_score_select_pages(const ekv_cache_desc* desc, const float* q, float scale,
                                  const void* K, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t refresh_last_page,
                                  int32_t top_k, void* kmin, void* kmax, float* ub,
                                  float* ubg, int32_t* sel, int32_t* n_sel, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* Counter bytes ekv_score_select_pages needs (0 if desc is invalid). */
size_t ekv_score_select_workspace_bytes(const ekv_cache_desc* desc);

/*
 * Top-k selection and sparse alpha-entmax decode in one call (§2.B(1) then
 * §2.C): the same sel, n_sel, out, tau_out and n_support as
 *   ekv_select_pages(TOPK, top_k, ubg)  ->
 *   ekv_entmax_decode(sel, n_sel, max_sel = min(top_k, max_pages_per_seq),
 *                     ub, zlb)
 * (ub NULL: without page pruning).  Where the shape allows (at most 1024
 * selected pages, max_pages_per_seq <= 8192) the selection runs inside the
 * decode's key launch: each of its workgroups selects the pair's pages itself
 * from ubg, probes each query head's best selected page for the pruning
 * bound, and scores an even share of the pages left to read; the selection
 * list never makes a round trip through memory before it is used.  Otherwise
 * the separate select and decode kernels run.  Two or three launches.
 * ubg [B][Hkv][maxP] and ub [B][Hkv][maxP][G] (16-byte aligned) as written by
 * ekv_score_pages or ekv_score_box_pages for the same query; hint: NULL, or
 * the hints ekv_score_box_pages wrote with them (used only with ub; a hint
 * buffer holding anything else only changes which selected page each head
 * probes, never the results: the probed page's physical page is taken from
 * block_table, and a page the top-k did not select is not used).  sel and
 * n_sel are outputs.
 * ws / ws_bytes: at least ekv_topk_decode_workspace_bytes(desc, top_k) bytes,
 * 256-byte aligned; no initialisation needed, garbage afterwards.
 */
ekv_status ekv_topk_decode(const ekv_cache_desc* desc, const float* q, float scale, float alpha,
                           const void* K, const void* V, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t top_k, const float* ub,
                           const float* ubg, const void* hint, int32_t* sel, int32_t* n_sel,
                           float* out, float* tau_out, int32_t* n_support, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/*
 * Box bounds only, the scoring of the top-k step (§2.A): ub and ubg exactly as
 * ekv_score_pages writes them (gm = gv = NULL), with each row's last page's
 * box first rebuilt from K when refresh_last_page is set (as
 * ekv_score_select_pages does; K may be NULL otherwise).  hint (or NULL):
 * ekv_score_hint_bytes(desc) bytes, 16-byte aligned, receive each page
 * slice's best page per query head; passed with ub to ekv_topk_decode for the
 * same query, they let each head's pruning probe be requested before the
 * selection runs (results unchanged).  Their content is internal to the
 * library.  One launch.
 */
ekv_status ekv_score_box_pages(const ekv_cache_desc* desc, const float* q, float scale,
                               const void* K, const int32_t* block_table,
                               const int32_t* seq_lens, int32_t refresh_last_page, void* kmin,
                               void* kmax, float* ub, float* ubg, void* hint,
                               hipStream_t stream);

/* Bytes of the best-page hints of ekv_score_box_pages (0 if desc is invalid). */
size_t ekv_score_hint_bytes(const ekv_cache_desc* desc);

/* Scratch bytes ekv_topk_decode needs (0 if desc is invalid or top_k < 1). */
size_t ekv_topk_decode_workspace_bytes(const ekv_cache_desc* desc, int32_t top_k);

/*
 * One whole decode step with the top-k policy (the pipeline of §2: scoring
 * from page metadata, candidate selection, sparse entmax over the selected
 * pages): ekv_score_box_pages with the per-head bounds and hints written to
 * the workspace (and, with refresh_last_page, each row's last page's box
 * rebuilt from K first), then ekv_topk_decode with page pruning on those
 * bounds; one workspace of ekv_step_workspace_bytes(desc,
 * top_k) bytes (zero-filled before first use, reusable afterwards).  With
 * refresh_last_page set, a row's last page must not be referenced by another
 * row.  The results equal those of ekv_score_select_pages followed by
 * ekv_entmax_decode with pruning.
 */
ekv_status ekv_decode_step(const ekv_cache_desc* desc, const float* q, float scale, float alpha,
                           const void* K, const void* V, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t refresh_last_page, int32_t top_k,
                           void* kmin, void* kmax, float* ubg, int32_t* sel, int32_t* n_sel,
                           float* out, float* tau_out, int32_t* n_support, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* Scratch bytes ekv_decode_step needs (0 if desc is invalid or top_k < 1). */
size_t ekv_step_workspace_bytes(const ekv_cache_desc* desc, int32_t top_k);

/*
 * ekv_decode_step for callers that cannot allocate device memory (code under
 * stream capture, serving loops and harnesses that forbid allocation): the
 * same arguments and results, minus ws / ws_bytes.  The step's scratch lives
 * in a device array of the library, EKV_NOALLOC_SCRATCH_BYTES bytes on each
 * GPU it runs on, held until the process ends: the arrival counters in its
 * first EKV_NOALLOC_COUNTER_BYTES (one int per (row, KV head) pair), the rest
 * of ekv_step_workspace_bytes(desc, top_k) after them.  A shape whose pairs or
 * scratch do not fit returns EKV_ERR_WORKSPACE before anything is launched;
 * nothing is allocated or freed.  The first call on a device looks up the
 * array's address on that device (with it current) and clears the counters
 * with a kernel on `stream`; every completed call leaves them zero.
 * All calls on one GPU share its array and keep the last call's contents:
 * calls that overlap in time on one GPU (different streams, or unordered host
 * threads) race on it and must not be issued.
 */
#define EKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
#define EKV_NOALLOC_COUNTER_BYTES ((size_t)64 << 10)
ekv_status ekv_decode_step_noalloc(const ekv_cache_desc* desc, const float* q, float scale,
                                   float alpha, const void* K, const void* V,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   int32_t refresh_last_page, int32_t top_k, void* kmin,
                                   void* kmax, float* ubg, int32_t* sel, int32_t* n_sel,
                                   float* out, float* tau_out, int32_t* n_support,
                                   hipStream_t stream);

/* Scratch bytes ekv_entmax_decode needs for this cache shape and max_sel
 * (0 if desc is invalid). */
size_t ekv_decode_workspace_bytes(const ekv_cache_desc* desc, int32_t max_sel);

/*
 * Softmax decode over the selected pages, or over every page of each row
 * (sel NULL): the comparison path of the EntmaxKV summary page (§3: under
 * softmax every token keeps positive weight, so dropping pages drops mass
 * delta > 0 and the output error is only bounded by 2 B delta; §4: the
 * method's speed is compared with a full-cache softmax decode of the
 * FlashDecoding kind).  For each row b and query head h (KV head g), over the
 * valid tokens i of the pages sel[b][g][0 .. n_sel[b][g]) (all pages
 * 0 .. n_b-1 when sel is NULL; entries are logical pages in [0, n_b), and an
 * entry outside that range is taken as a page with no valid token):
 *   s_i = scale * <q[b][h], k_i>                         (fp32 accumulation)
 *   out[b][h] = sum_i exp(s_i) v_i / sum_i exp(s_i)      (fp32, every value
 *                                                          row is read)
 *   lse[b][h] = ln sum_i exp(s_i)  (fp32, [B][Hq]), if lse is not NULL.
 * The dropped softmax mass of a selection is 1 - exp(lse_sel - lse_all),
 * with lse_all from the call with sel NULL.  An empty row (or n_sel 0) gets a
 * zero output and lse = -inf; a row whose n_sel exceeds max_sel gets NaN.
 * max_sel: host upper bound on every n_sel[b][g] (<= 0, or sel NULL: the
 *   row capacity max_pages_per_seq); it sizes the launch and the workspace.
 * ws / ws_bytes: device scratch of at least ekv_softmax_workspace_bytes(desc,
 *   max_sel) bytes, 256-byte aligned; no initialisation needed, garbage
 *   afterwards.  scale > 0 and finite.  Two launches (split partials, merge).
 */
ekv_status ekv_softmax_decode(const ekv_cache_desc* desc, const float* q, float scale,
                              const void* K, const void* V, const int32_t* block_table,
                              const int32_t* seq_lens, const int32_t* sel,
                              const int32_t* n_sel, int32_t max_sel, float* out, float* lse,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* Scratch bytes ekv_softmax_decode needs for this cache shape and max_sel
 * (0 if desc is invalid; pass max_sel <= 0 for the full-cache call). */
size_t ekv_softmax_workspace_bytes(const ekv_cache_desc* desc, int32_t max_sel);

/* e_n = E[max of n iid N(0,1)] as used by EKV_SELECT_GAUSS_EST for a page of
 * n valid tokens (tabulated once on the host by quadrature); NaN unless
 * 1 <= n <= 64.  Host-only: launches nothing, needs no device. */
double ekv_gauss_expected_max(int32_t n);

/* Static description of a status code (never NULL). */
const char* ekv_status_string(ekv_status status);

#ifdef __cplusplus
}
#endif

#endif /* ENTMAXKV_H */
