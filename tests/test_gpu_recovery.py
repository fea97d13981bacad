"""GPU: failure in the middle of a chunk-causal rollout, and the retry.

A streaming caller keeps the last committed state and hands it to the next
chunk (SANA-Video talk, block cache: cache the state, add the next block).
When one chunk's call fails its checks, nothing may have been written: the
committed state must be exactly what it was, so that the caller can retry
the chunk from it.  The rollout with failures and retries must give bitwise
the outputs and final state of the uninterrupted rollout.
"""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import frame_wise_gated_gdn_amd as gdn
    from frame_wise_gated_gdn_amd import workloads
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    gdn.lib()
    return torch, gdn, workloads


def chunks_of(inp, T, c):
    return [tuple(inp[n][:, :, t0:min(T, t0 + c)].contiguous() for n in ("q", "k", "v", "gamma", "beta"))
            for t0 in range(0, T, c)]


@pytest.mark.parametrize("path", ["auto", "one_launch"])
def test_failed_chunks_leave_the_state_and_retry_gives_the_same_rollout(env, path):
    torch, gdn, wl = env
    w = wl.CHUNKED
    inp = wl.generate(w, device="cuda")
    B, H, D = w.B, w.H, w.D
    chunks = chunks_of(inp, w.T, w.chunk)

    state_ref = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
    outs_ref = []
    for ch in chunks:
        o, _, _ = gdn.frame_step(*ch, state_ref, commit="inplace", path=path)
        outs_ref.append(o)
    torch.cuda.synchronize()

    fail_ws, fail_alias, fail_shape = 3, 11, len(chunks) - 1     # chunks whose first call fails
    state = torch.zeros_like(state_ref)
    outs = []
    for i, ch in enumerate(chunks):
        if i in (fail_ws, fail_alias, fail_shape):
            before = state.clone()
            out = torch.full_like(ch[0], 7.0)
            out_before = out.clone()
            if i == fail_ws:
                # a workspace too small for even one frame
                bad = torch.empty(16, dtype=torch.uint8, device="cuda")
                with pytest.raises(gdn.GDNError) as e:
                    gdn.frame_step(*ch, state, out=out, commit="inplace", workspace=bad, path=path)
                assert e.value.status == 8, e.value          # GDN_ERR_WORKSPACE
            elif i == fail_alias:
                # the output aliases the queries
                q_before = ch[0].clone()
                with pytest.raises(gdn.GDNError) as e:
                    gdn.frame_step(*ch, state, out=ch[0], commit="inplace", path=path)
                assert e.value.status == 5, e.value          # GDN_ERR_ALIAS
                torch.cuda.synchronize()
                assert torch.equal(ch[0], q_before), "a failed chunk wrote over its queries"
            else:
                # an output that is not 16-byte aligned
                raw = torch.full((ch[0].numel() + 1,), 7.0, dtype=ch[0].dtype, device="cuda")
                odd = raw[1:].view(ch[0].shape)
                with pytest.raises(gdn.GDNError) as e:
                    gdn.frame_step(*ch, state, out=odd, commit="inplace", path=path)
                assert e.value.status == 4, e.value          # GDN_ERR_ALIGN
                assert torch.equal(odd, out_before), "a failed chunk wrote its output"
            torch.cuda.synchronize()
            assert torch.equal(state, before), "a failed chunk changed the committed state"
            assert torch.equal(out, out_before), "a failed chunk wrote its output"
            # retry the same chunk from the same committed state
            o, _, _ = gdn.frame_step(*ch, state, out=out, commit="inplace", path=path)
        else:
            o, _, _ = gdn.frame_step(*ch, state, commit="inplace", path=path)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, dim=2), torch.cat(outs_ref, dim=2))
    assert torch.equal(state, state_ref)
