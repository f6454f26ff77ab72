/*
 * msa.h -- C ABI of the MiniMax Sparse Attention (MSA) forward path for AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed (Sparse Attention Part II, mtreviso.github.io, section 3.2
 * "MiniMax's MSA"; MiniMax Sparse Attention, api.staik.se blog): for every
 * query and GQA group an index query is scored against one index key head
 * shared by all groups, over the causally visible tokens.  Each block of
 * `block_size` key tokens is scored by the maximum of its token scores.  A
 * Top-k over the block scores keeps `topk` blocks per query and group, one of
 * them always the query's own (local) block.  Every query head of the group
 * then runs exact attention over the visible tokens of the kept blocks, with
 * its own softmax normalised over that set only.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers, allocated and owned by the
 *     caller.  The library never allocates, frees or synchronises; it keeps no
 *     mutable global state, so calls on different streams may run
 *     concurrently.  `stream` is a hipStream_t (NULL = the null stream).
 *   - Layouts are dense, row-major, with no padding ("BSHD"):
 *       q      [B][S_q][H_q][D]       bf16
 *       k, v   [B][S_k][H_kv][D]      bf16
 *       q_idx  [B][S_q][H_kv][D_idx]  bf16  (one index-query head per group)
 *       k_idx  [B][S_k][D_idx]        bf16  (one index-key head, shared)
 *       block_scores [B][H_kv][S_q][n_blk] fp32, n_blk = ceil(S_k / block_size)
 *       block_idx    [B][H_kv][S_q][topk]  int32
 *       out    [B][S_q][H_q][D]       bf16
 *       lse    [B][H_q][S_q]          fp32 (natural log), optional
 *   - Query i sits at absolute position t_i = i + S_k - S_q (the queries are
 *     the last S_q positions of the key sequence; decode is S_q = 1).  Its
 *     local block is l_i = floor(t_i / block_size).  Query head h belongs to
 *     group g = floor(h / (H_q / H_kv)).
 *   - All pointers must be 16-byte aligned.
 *   - Argument checks run on the host before any HIP call; a failed check
 *     returns its status and launches nothing.  A HIP launch error returns
 *     MSA_ERR_HIP.  Faults inside kernels surface at the caller's next
 *     synchronisation, as for any asynchronous HIP work.
 *   - Results are bit-identical from run to run (for the same ws_bytes).
 *   - Workspace: an entry point that takes `ws` accepts any ws_bytes from
 *     msa_workspace_min_bytes(dims, entry) up; msa_workspace_bytes(dims,
 *     entry) is the size it is designed for.  The entries that keep per-edge
 *     records (the attention forward, msa_forward, both backward entries) run
 *     the queries in the largest chunks whose workspace fits ws_bytes, never
 *     larger than with msa_workspace_bytes (whole 128-query blocks from 128
 *     queries on; msa_attn_chunks counts them).  Smaller workspaces give the
 *     same forward results; the backward's key gradients are then summed
 *     across chunks in fp32, so their last bits may depend on ws_bytes.
 *   - batch == 0 or seqlen_q == 0 is an empty problem: MSA_OK, no launch
 *     (except msa_kl_loss_fwd, which writes its loss of 0).
 *
 * Supported on this device path: causal = 1, head_dim = 128,
 * index_dim in {64, 128}, block_size = 128, 1 <= topk <= 64,
 * seqlen_k >= seqlen_q, num_heads_q a multiple of num_heads_kv with
 * H_q / H_kv in {1, 2, 4, 8, 16, 32}.  Other values return
 * MSA_ERR_UNSUPPORTED (or MSA_ERR_INVALID_DIMS when they are not meaningful).
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum msa_status {
  MSA_OK = 0,
  MSA_ERR_NULL_PTR = 1,           /* a required pointer is NULL */
  MSA_ERR_INVALID_DIMS = 2,       /* negative sizes or scale, S_k < S_q, H_q % H_kv != 0, ... */
  MSA_ERR_UNSUPPORTED = 3,        /* meaningful, but outside the device path's set */
  MSA_ERR_MISALIGNED = 4,         /* a pointer is not 16-byte aligned */
  MSA_ERR_WORKSPACE_TOO_SMALL = 5,/* ws_bytes < msa_workspace_min_bytes(...) */
  MSA_ERR_HIP = 6                 /* a HIP runtime call or launch failed */
} msa_status;

typedef struct msa_dims {
  int32_t batch;         /* B */
  int32_t seqlen_q;      /* S_q: new queries per sequence */
  int32_t seqlen_k;      /* S_k: keys per sequence (prefix incl. the queries) */
  int32_t num_heads_q;   /* H_q: main-branch query heads */
  int32_t num_heads_kv;  /* H_kv: KV heads = GQA groups = index-query heads */
  int32_t head_dim;      /* D */
  int32_t index_dim;     /* D_idx: width of the index query / key */
  int32_t block_size;    /* key tokens per block */
  int32_t topk;          /* blocks kept per query and group, local block incl. */
  int32_t causal;        /* must be 1 */
  float softmax_scale;   /* main-branch logit scale (>= 0); 0 selects 1/sqrt(D) */
} msa_dims;

/* Which call a workspace size is asked for. */
typedef enum msa_entry {
  MSA_ENTRY_INDEX_SCORES = 0,
  MSA_ENTRY_BLOCK_TOPK = 1,
  MSA_ENTRY_SPARSE_ATTN_FWD = 2,
  MSA_ENTRY_FORWARD = 3,
  MSA_ENTRY_KL_LOSS_FWD = 4,
  MSA_ENTRY_SPARSE_ATTN_BWD = 5,
  MSA_ENTRY_KL_LOSS_BWD = 6,
  MSA_ENTRY_BACKWARD = 7
} msa_entry;

/*
 * Index branch, scoring step (section 3.2 of Sparse Attention Part II: the
 * index query is dotted with the one index key all groups share, over the
 * causally visible keys, and
 * each block is scored by its maximum token score; section 4.4 of the same
 * page for keeping the token scores off HBM).
 *
 *   block_scores[b][g][i][j] = max over s in block j with s <= t_i of
 *                              sum_c q_idx[b][i][g][c] * k_idx[b][s][c]
 *   and -infinity for blocks j > l_i (nothing visible).
 *
 * The raw dot product is used: no scale and no activation.  Products are
 * exact in fp32 and sums accumulate in fp32 on the matrix cores, so the
 * result is exact whenever every partial sum is an integer below 2^24 (as
 * with small integer-valued inputs).  Token scores are never written to
 * memory.  Inputs: q_idx, k_idx (read only).  Output: block_scores (written
 * in full, including the -infinity entries).
 */
msa_status msa_index_scores(const msa_dims* dims, const void* q_idx,
                            const void* k_idx, float* block_scores,
                            void* stream);

/*
 * Index branch, selection step (section 3.2 of Sparse Attention Part II: one
 * of the k slots is reserved for the query's local block and the indexer
 * picks the others; the MiniMax Sparse Attention blog: the Top-k works on raw
 * scores, with no exponential; section 4.2 of Sparse Attention Part II: exact
 * top-k must break equal scores in one fixed way).
 *
 *   Sel_i = { l_i } united with the (topk - 1) best blocks among 0 .. l_i - 1,
 *           ranked by block score (higher first) and, on equal scores, by
 *           block index (lower first); all of 0 .. l_i - 1 when l_i < topk.
 *
 *   block_idx[b][g][i][0 .. n-1] = Sel_i in ascending order, n = min(topk, l_i + 1),
 *   block_idx[b][g][i][n .. topk-1] = -1.
 *
 * The local block's own score is not ranked.  Input: block_scores as written
 * by msa_index_scores (finite for j < l_i; NaN is not supported).  Output:
 * block_idx (written in full).
 */
msa_status msa_block_topk(const msa_dims* dims, const float* block_scores,
                          int32_t* block_idx, void* stream);

/*
 * Main branch (section 3.2 of Sparse Attention Part II: every query head of
 * the group attends to the causally visible tokens of the selected blocks
 * with its own weights; section 2 of the same page: the softmax is normalised
 * within the selection; section 4.1: O = P V with P the softmax of the scaled
 * scores, computed tile by tile without storing P).
 *
 *   T_i = { s : floor(s / block_size) in block_idx[b][g][i][:], s <= t_i }
 *   out[b][i][h] = sum_{s in T_i} softmax_s(scale * q[b][i][h] . k[b][s][g]) v[b][s][g]
 *   lse[b][h][i] = log sum_{s in T_i} exp(scale * q[b][i][h] . k[b][s][g])
 *
 * Entries of block_idx equal to -1 are ignored; the others must be distinct,
 * lie in 0 .. l_i, and include l_i (as msa_block_topk writes them).  Inputs
 * q, k, v, block_idx are read only.  `lse` may be NULL.  `ws` is scratch of at
 * least msa_workspace_min_bytes(dims, MSA_ENTRY_SPARSE_ATTN_FWD) bytes (see
 * the workspace convention above), owned by the caller; its contents on entry
 * do not matter and are clobbered.
 */
msa_status msa_sparse_attn_fwd(const msa_dims* dims, const void* q,
                               const void* k, const void* v,
                               const int32_t* block_idx, void* out, float* lse,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * The whole forward path in the order the pages give it (The Architecture of
 * Infinity, baystreetwire.com: index/proxy attention first, then the sparse
 * main attention; Sparse Attention Part II, section 3.2 figure: hidden states,
 * indexer scores, selected indices, main attention): msa_index_scores, then
 * msa_block_topk, then msa_sparse_attn_fwd, all on `stream`, with the block
 * scores kept in `ws`.  When topk <= 16 and seqlen_q * num_heads_kv > 32 the
 * first two run as one kernel that keeps each row's running Top-k in
 * registers and never writes the block scores (same selection, bit for bit).
 * `block_idx_out` (may be NULL) receives the selection; `lse` may be NULL.
 * `ws` must hold at least msa_workspace_min_bytes(dims, MSA_ENTRY_FORWARD)
 * bytes: the block scores (when they are written), the selection, then the
 * attention's workspace in the rest.
 */
msa_status msa_forward(const msa_dims* dims, const void* q, const void* k,
                       const void* v, const void* q_idx, const void* k_idx,
                       void* out, float* lse, int32_t* block_idx_out, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * msa_forward for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same
 * computation and results as msa_forward, with the workspace taken from a
 * static device array inside the library instead of the caller.  The array
 * holds MSA_NOALLOC_SCRATCH_BYTES bytes on each GPU the call runs on (the
 * current device; `stream` must belong to it), from the first call there
 * until the process ends; the attention runs in as many query chunks as that
 * size requires.  The call allocates and frees nothing.  A problem whose
 * smallest workspace (msa_workspace_min_bytes(dims, MSA_ENTRY_FORWARD)) is
 * larger returns MSA_ERR_WORKSPACE_TOO_SMALL and launches nothing.  All
 * calls on one GPU share the array: calls that overlap on one GPU (several
 * streams or host threads) race and must be serialised by the caller.
 * Arguments, checks and errors otherwise as msa_forward; MSA_ERR_HIP also if
 * the array's address cannot be obtained.
 */
#define MSA_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
msa_status msa_forward_noalloc(const msa_dims* dims, const void* q, const void* k,
                               const void* v, const void* q_idx, const void* k_idx,
                               void* out, float* lse, int32_t* block_idx_out,
                               void* stream);

/*
 * Block-mask form of a selection (Sparse Attention Part II, section 4.3: the
 * blocks a query visits kept as one flag per block, 32 flags to an unsigned
 * word, block j at bit j mod 32 of word floor(j / 32)):
 *
 *   mask[b][g][i][w], w < ceil(n_blk / 32), n_blk = ceil(seqlen_k / block_size):
 *   bit j mod 32 of word floor(j / 32) is 1 iff j appears in block_idx[b][g][i][0 .. topk-1].
 *
 * Entries equal to -1, or outside 0 .. n_blk-1, set nothing; bits past the
 * last block are 0.  Storage: 4 * ceil(n_blk / 32) bytes per row.  Uses the
 * dims' batch, seqlen_q, seqlen_k, num_heads_kv, block_size (128) and topk.
 * Pointers are device pointers, 16-byte aligned; the call allocates nothing.
 */
msa_status msa_block_mask(const msa_dims* dims, const int32_t* block_idx,
                          uint32_t* mask, void* stream);

/*
 * The traversal of the same section: for each row, walk the words in order;
 * a word's popcount is its number of active blocks and the position of its
 * rank-th set bit gives block 32 w + bit.  block_idx[b][g][i][0 .. topk-1]
 * receives the blocks in ascending order, at most topk of them (the lowest
 * ones when a row has more), then -1.  Bits past the last block are ignored.
 * Same layouts and dims as msa_block_mask.
 */
msa_status msa_mask_blocks(const msa_dims* dims, const uint32_t* mask,
                           int32_t* block_idx, void* stream);

/*
 * Alignment loss of the index branch, forward value (Sparse Attention Part
 * II, section 3.2: after the dense warm-up, the index projections are trained
 * by a KL term over the tokens of the selected blocks; the target is the
 * group's mean main-branch distribution and is not differentiated).  For row
 * (b, g, i) with T_i as in msa_sparse_attn_fwd:
 *
 *   P(s)    = (1/G) sum_{h in group g} exp(scale * q[b][i][h] . k[b][s][g] - lse[b][h][i])
 *   Pidx(s) = softmax over s in T_i of z(s) = q_idx[b][i][g] . k_idx[b][s]
 *   kl_rows[b][g][i] = sum_{s in T_i} P(s) ln(P(s) / Pidx(s))
 *   *loss = (1 / (B * S_q * H_kv)) * sum of kl_rows
 *
 * G = H_q / H_kv.  The index score z is the raw dot product (no scale), the
 * same token score that msa_index_scores max-pools.  `lse` is the main
 * branch's log-sum-exp over the same selection, exactly as msa_forward or
 * msa_sparse_attn_fwd return it ([B][H_q][S_q], natural log); it normalises
 * each head's probabilities on T_i, so neither distribution is formed in
 * memory.  block_idx follows the rules of msa_sparse_attn_fwd.  kl_rows
 * ([B][H_kv][S_q] fp32) and loss (one fp32) are each optional (NULL skips
 * it); the loss is summed in a fixed order, so it is identical from run to
 * run.  lse_idx ([B][H_kv][S_q] fp32, optional) receives each row's
 * log-sum-exp of z over T_i, which msa_kl_loss_bwd takes.  `ws` holds
 * msa_workspace_bytes(dims, MSA_ENTRY_KL_LOSS_FWD) bytes
 * (edge lists and 32 bytes per selected block per row); contents on entry do
 * not matter.  An empty problem writes *loss = 0 when loss is not NULL.
 * Uses every field of dims (both branches).
 */
msa_status msa_kl_loss_fwd(const msa_dims* dims, const void* q, const void* k,
                           const void* q_idx, const void* k_idx,
                           const int32_t* block_idx, const float* lse,
                           float* kl_rows, float* loss, float* lse_idx,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * Main branch, backward (the backward pass that the MSA kernel notes fuse
 * over the selected blocks, The Architecture of Infinity, baystreetwire.com;
 * Sparse Attention Part II, section 2: inside the selection the attention is
 * an ordinary softmax attention over the selected tokens).  The selection is
 * a discrete choice and carries no gradient.  For each head h of group g,
 * with P_s = exp(scale * q[b][i][h] . k[b][s][g] - lse[b][h][i]) on T_i and
 * Delta = sum_d dout[b][i][h][d] * out[b][i][h][d]:
 *
 *   dS_s = P_s (dout[b][i][h] . v[b][s][g] - Delta)
 *   dq[b][i][h] = scale * sum_{s in T_i} dS_s k[b][s][g]
 *   dk[b][s][g] = scale * sum over (i, h in g) with s in T_i of dS_s q[b][i][h]
 *   dv[b][s][g] = sum over (i, h in g) with s in T_i of P_s dout[b][i][h]
 *
 * Inputs: q, k, v, block_idx (as msa_sparse_attn_fwd), out and lse exactly as
 * the forward returned them for this selection, dout [B][S_q][H_q][D] bf16.
 * Outputs (written in full, bf16): dq like q; dk, dv like k and v (zero for
 * keys no query selects; an empty problem with batch > 0 writes dk = dv = 0).
 * Sums run in a fixed order: results are identical
 * from run to run for the same ws_bytes.  `ws` holds at least
 * msa_workspace_min_bytes(dims, MSA_ENTRY_SPARSE_ATTN_BWD) bytes (edge lists,
 * per-edge dq records of G * (3 D / 2 + 16) bytes per chunk, fp32 dk / dv
 * parts of the key blocks so many queries select that their gradient is
 * split over several workgroups, 128 KiB per part, and fp32 dk / dv sums
 * when the queries run in several chunks); contents on entry do not
 * matter.  Uses the main-branch fields of
 * dims (index_dim is ignored).
 */
msa_status msa_sparse_attn_bwd(const msa_dims* dims, const void* q, const void* k,
                               const void* v, const int32_t* block_idx,
                               const void* out, const float* lse, const void* dout,
                               void* dq, void* dk, void* dv, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * Alignment loss, backward: the gradient of grad_loss * loss (loss as
 * msa_kl_loss_fwd defines it) with respect to the index inputs.  The teacher
 * is detached (Sparse Attention Part II, section 3.2), so q, k get nothing
 * from this loss; the KL expansion (The Architecture of Infinity) makes the
 * gradient of each index score z(s) of row (b, g, i), for s in T_i,
 *
 *   g(s) = grad_loss / (B * S_q * H_kv) * (exp(z(s) - lse_idx[b][g][i]) - P(s))
 *   dq_idx[b][i][g] = sum_{s in T_i} g(s) k_idx[b][s]
 *   dk_idx[b][s]    = sum over rows (b, g, i) with s in T_i of g(s) q_idx[b][i][g]
 *
 * with P the teacher of msa_kl_loss_fwd.  Inputs as msa_kl_loss_fwd, plus
 * lse_idx as that call wrote it for the same selection.  Outputs bf16, written
 * in full: dq_idx like q_idx, dk_idx like k_idx (zero for keys no row
 * selects; an empty problem with batch > 0 writes dk_idx = 0).  Fixed
 * summation order: identical from run to run.  `ws` holds at least
 * msa_workspace_min_bytes(dims, MSA_ENTRY_KL_LOSS_BWD) bytes (edge lists,
 * 2 D_idx + 16 bytes per selected block per row of a query chunk, and fp32
 * dk_idx per group).
 */
msa_status msa_kl_loss_bwd(const msa_dims* dims, const void* q, const void* k,
                           const void* q_idx, const void* k_idx,
                           const int32_t* block_idx, const float* lse,
                           const float* lse_idx, float grad_loss, void* dq_idx,
                           void* dk_idx, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole backward in one call: msa_sparse_attn_bwd and msa_kl_loss_bwd
 * over the same selection (the MSA kernel notes pair the proxy's backward
 * with the main backward because the proxy's signal needs both probability
 * sets, The Architecture of Infinity, baystreetwire.com; Sparse Attention
 * Part II, section 3.2 for the loss).  Each query chunk's edge buckets are
 * built and sorted once and serve both passes: dq, dk, dv as
 * msa_sparse_attn_bwd defines them, and dq_idx, dk_idx (the gradient of
 * grad_loss * loss) as msa_kl_loss_bwd does.  Inputs: q, k, v, q_idx, k_idx,
 * block_idx as msa_forward; out and lse as the forward returned them; lse_idx
 * as msa_kl_loss_fwd wrote it for the same selection; dout [B][S_q][H_q][D]
 * bf16.  Outputs bf16, written in full: dq like q, dk and dv like k and v,
 * dq_idx like q_idx, dk_idx like k_idx; when this call and the separate ones
 * each run in one query chunk, every output equals the separate entry
 * point's bit for bit (same kernels, same summation orders).  `ws` holds at
 * least msa_workspace_min_bytes(dims, MSA_ENTRY_BACKWARD) bytes (both passes'
 * per-edge records); contents on entry do not matter.  Errors as the two
 * separate calls.
 */
msa_status msa_backward(const msa_dims* dims, const void* q, const void* k, const void* v,
                        const void* q_idx, const void* k_idx, const int32_t* block_idx,
                        const void* out, const float* lse, const float* lse_idx,
                        const void* dout, float grad_loss, void* dq, void* dk, void* dv,
                        void* dq_idx, void* dk_idx, void* ws, size_t ws_bytes, void* stream);

/* Internal stages of msa_forward, in launch order (for msa_forward_profiled). */
typedef enum msa_stage {
  MSA_STAGE_INDEX_SCORES = 0,  /* index scores fused with the block max-pool */
  MSA_STAGE_BLOCK_TOPK = 1,    /* exp-free Top-k */
  MSA_STAGE_ATTN_BUILD = 2,    /* edges grouped by (batch, group, block) */
  MSA_STAGE_ATTN_PARTIAL = 3,  /* attention of each edge over its block */
  MSA_STAGE_ATTN_MERGE = 4,    /* per-query merge of the partial results */
  MSA_N_STAGES = 5
} msa_stage;

/*
 * msa_forward with timing instrumentation, for profilers and benchmarks (the
 * tracing hooks of the forward path; same arguments, same results).  `events`
 * holds n_events caller-created hipEvent_t handles, all recorded on `stream`:
 *   events[0], events[1]   before and after the index scores
 *                          (MSA_STAGE_INDEX_SCORES; with the fused selection
 *                          this pair covers the Top-k too)
 *   events[2], events[3]   before and after the Top-k (MSA_STAGE_BLOCK_TOPK;
 *                          an empty pair with the fused selection)
 *   events[4 + 6 c + 2 m], events[4 + 6 c + 2 m + 1]
 *                          before and after stage MSA_STAGE_ATTN_BUILD + m
 *                          (m = 0, 1, 2) of query chunk c, c = 0 .. chunks-1
 * where chunks = msa_attn_chunks(dims, MSA_ENTRY_FORWARD, ws_bytes).  Returns
 * MSA_ERR_NULL_PTR if events is NULL or holds a NULL handle, and
 * MSA_ERR_INVALID_DIMS if n_events < 4 + 6 * chunks.
 */
msa_status msa_forward_profiled(const msa_dims* dims, const void* q, const void* k,
                                const void* v, const void* q_idx, const void* k_idx,
                                void* out, float* lse, int32_t* block_idx_out,
                                void* ws, size_t ws_bytes, void* stream,
                                void* const* events, int n_events);

/*
 * Number of query chunks the entry point runs in with a workspace of ws_bytes
 * (see the workspace convention above): 1 or more for the entries that take a
 * workspace (always 1 for MSA_ENTRY_KL_LOSS_FWD); 0 for invalid dims, an
 * empty problem, ws_bytes below msa_workspace_min_bytes, or an entry without
 * a workspace.
 */
int msa_attn_chunks(const msa_dims* dims, int entry, size_t ws_bytes);

/*
 * Bytes of caller-provided workspace the given entry point is designed for
 * with these dims (0 for entries that need none): its query chunks keep at
 * most 48 GiB of per-edge records.  Returns (size_t)-1 when the dims are not
 * valid for that entry point.
 */
size_t msa_workspace_bytes(const msa_dims* dims, int entry);

/*
 * The smallest workspace the entry point accepts for these dims (one query
 * per chunk); below it the call returns MSA_ERR_WORKSPACE_TOO_SMALL.
 * (size_t)-1 when the dims are not valid for that entry point.
 */
size_t msa_workspace_min_bytes(const msa_dims* dims, int entry);

/* Static, human-readable name of a status code. */
const char* msa_status_str(msa_status status);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
