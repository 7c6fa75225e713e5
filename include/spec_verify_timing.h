/*
 * spec_verify_timing.h -- instrumented twins of the entry points of
 * spec_verify.h, for benchmark timing only.
 *
 * Each *_timed function takes the same arguments as the entry point of the
 * same name, does the same work with the same kernels and results, and takes
 * one more argument:
 *
 *  phase_events  NULLABLE array of hipEvent_t handles created with timing
 *                enabled.  [0] and [1] are recorded by the launch of the
 *                kernel that streams every logit once (the row-statistics
 *                pass of chains, stochastic trees, outcome scoring and tree
 *                construction; the row-argmax pass of greedy tree
 *                verification), at that kernel's start and end, on `stream`.
 *                For spec_verify_chain_timed, spec_verify_chain_pointmass_timed
 *                and spec_verify_tree_stochastic_timed, [2] is recorded on
 *                `stream` after the final-draw kernels (before the optional
 *                final_dist pass).  NULL behaves as the product entry point.
 *
 * Errors, ownership and asynchrony are those of the product entry points; an
 * event that cannot be recorded returns SV_ERR_HIP.
 */
#ifndef SPEC_VERIFY_TIMING_H
#define SPEC_VERIFY_TIMING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int32_t spec_verify_chain_timed(const void *target_logits, const void *draft_logits,
                                int32_t dtype, const int32_t *draft_tokens,
                                const float *uniforms, int32_t B, int32_t gamma, int32_t V,
                                double temperature, int32_t *accept_len, int32_t *out_tokens,
                                float *final_dist, void *workspace, size_t workspace_bytes,
                                void *stream, void *const *phase_events);

int32_t spec_verify_chain_pointmass_timed(const void *target_logits, int32_t dtype,
                                          const int32_t *draft_tokens, const float *uniforms,
                                          int32_t B, int32_t gamma, int32_t V,
                                          double temperature, int32_t *accept_len,
                                          int32_t *out_tokens, float *final_dist,
                                          void *workspace, size_t workspace_bytes, void *stream,
                                          void *const *phase_events);

int32_t spec_verify_tree_greedy_timed(const void *target_logits, int32_t dtype,
                                      const int32_t *parents, const int32_t *tokens, int32_t B,
                                      int32_t n, int32_t V, int32_t *accept_len,
                                      int32_t *accept_node, int32_t *out_tokens, void *workspace,
                                      size_t workspace_bytes, void *stream,
                                      void *const *phase_events);

int32_t spec_verify_tree_stochastic_timed(const void *target_logits, const void *draft_logits,
                                          int32_t dtype, const int32_t *parents,
                                          const int32_t *tokens, const float *uniforms,
                                          int32_t B, int32_t n, int32_t V, double temperature,
                                          int32_t *accept_len, int32_t *accept_node,
                                          int32_t *out_tokens, float *final_dist,
                                          void *workspace, size_t workspace_bytes, void *stream,
                                          void *const *phase_events);

int32_t spec_outcome_topk_timed(const void *logits, int32_t dtype, const int32_t *draft_tokens,
                                int32_t R, int32_t gamma, int32_t V, double temperature,
                                int32_t ncache, int32_t *out_k, int32_t *out_a, double *out_p,
                                double *hit, void *workspace, size_t workspace_bytes,
                                void *stream, void *const *phase_events);

int32_t spec_tree_build_timed(const void *draft_logits, int32_t dtype, const int32_t *child_row,
                              int32_t R, int32_t M, int32_t V, double temperature, int32_t W,
                              int32_t max_depth, int32_t budget, int32_t *parents,
                              int32_t *tokens, int32_t *node_row, double *score,
                              int32_t *n_nodes, void *workspace, size_t workspace_bytes,
                              void *stream, void *const *phase_events);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_TIMING_H */
