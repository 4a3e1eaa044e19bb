"""The binding refuses tensors whose sizes do not match what it tells the library: the
library addresses every buffer by the shapes it is given, so a smaller tensor would be read
or written out of bounds.  CPU: the two checks themselves.  GPU: every entry point refuses
a mismatched tensor before anything is launched (tiny shapes; the well-formed calls run)."""
from __future__ import annotations

import pytest
import torch

import precision_attention_input_amd as ulp


def test_need_checks_elements_and_dtype():
    ulp._need(None, (3, 3), ulp._F32, "x")
    ulp._need(torch.empty(3, 3), (3, 3), ulp._F32, "x")
    ulp._need(torch.empty(9), (3, 3), ulp._F32, "x")          # same elements, other view
    with pytest.raises(ValueError, match="9 elements"):
        ulp._need(torch.empty(2, 3), (3, 3), ulp._F32, "x")
    with pytest.raises(ValueError, match="float32"):
        ulp._need(torch.empty(3, 3, dtype=torch.float16), (3, 3), ulp._F32, "x")


def test_need_bytes_measures_the_storage_from_the_view():
    g = torch.empty(4, 4, 1000, dtype=torch.uint8)
    ulp._need_bytes(g[0, 1], 3 * 4 * 1000 + 1000, "send")     # reaches g[3, 1] through a stride
    ulp._need_bytes(g[3, 2], 2000, "send")                     # exactly to the end
    with pytest.raises(ValueError, match="2001"):
        ulp._need_bytes(g[3, 2], 2001, "send")


@pytest.mark.gpu
def test_entry_points_refuse_mismatched_tensors(olib):
    dev = torch.device("cuda:0")
    P, B, L, H, D = 2, 1, 64, 4, 64
    h = H // P
    x = lambda *s: torch.randn(*s, device=dev).to(torch.bfloat16)
    q, k, v = x(B, L, H, D), x(B, L, H, D), x(B, L, H, D)
    mean = x(B, H, D)
    qa = ulp.k_grouped_amax(q, None, rank=0, world_size=P)
    ka = ulp.k_grouped_amax(k, mean, rank=0, world_size=P)
    with pytest.raises(ValueError, match="k_mean_global"):
        ulp.k_grouped_amax(k, x(B, H, D - 1), rank=0, world_size=P)
    with pytest.raises(ValueError, match="out"):
        ulp.k_grouped_amax(k, mean, rank=0, world_size=P,
                           out=torch.empty(B, H, 2, device=dev))
    with pytest.raises(ValueError, match="gathered_minmax"):
        ulp.derive_k_boundary_amax(ka, torch.empty(1, B, H, 2, 2, D, device=dev), mean,
                                   rank=0, local_sequence=L, world_size=P)
    with pytest.raises(ValueError, match="v"):
        ulp.pack(q, k, x(B, L - 1, H, D), mean, qa, ka, rank=0, world_size=P)
    with pytest.raises(ValueError, match="k_amax"):
        ulp.pack(q, k, v, mean, qa, ka[:, :1].contiguous(), rank=0, world_size=P)
    send = ulp.pack(q, k, v, mean, qa, ka, rank=0, world_size=P)
    with pytest.raises(ValueError, match="send"):
        ulp.pack(q, k, v, mean, qa, ka, rank=0, world_size=P, send=send[1],
                 dest_stride=send.shape[1])
    with pytest.raises(ValueError, match="recv_u8"):
        ulp.unpack_for_sage(send[:, :-256].contiguous(), batch_size=B, local_sequence=L,
                            local_heads=h, head_dim=D, world_size=P)
    outs = ulp.unpack_for_sage(send, batch_size=B, local_sequence=L, local_heads=h,
                               head_dim=D, world_size=P)
    bad = list(outs)
    bad[2] = torch.empty(B, D, h, 64 * P - 64, dtype=torch.uint8, device=dev)
    with pytest.raises(ValueError, match="v8"):
        ulp.unpack_for_sage(send, batch_size=B, local_sequence=L, local_heads=h, head_dim=D,
                            world_size=P, out=tuple(bad))
    q8, k8, v8, qs, ks = outs
    with pytest.raises(ValueError, match="k8"):
        ulp.consumer_attention(q8, k8[:, :-1].contiguous(), v8, qs, ks, used=L * P)
    with pytest.raises(ValueError, match="k_scale"):
        ulp.consumer_attention(q8, k8, v8, qs, ks[..., :-1].contiguous(), used=L * P)
    st = torch.stack
    with pytest.raises(ValueError, match="ranks"):
        ulp.group_stats(st([q, q]), st([k, k]), mean, world_size=4)
    with pytest.raises(ValueError, match="group"):
        ulp.group_pack(st([q, q]), st([k, k]), st([v, v]), mean, st([qa, qa]), st([ka, ka]),
                       world_size=P, group=torch.empty(P, P, 256, dtype=torch.uint8,
                                                       device=dev))
    with pytest.raises(ValueError, match="mean_dtype"):
        ulp.k_mean(st([k, k]), world_size=P,
                   out=(torch.empty(B, H, D, device=dev),
                        torch.empty(B, H, D, dtype=torch.float16, device=dev)))
    torch.cuda.synchronize()
